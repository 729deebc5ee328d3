"""One rank's context-parallel contract, composed across calls on one GPU.

The 32768-token lognormal batch of the sharded workload is run as its eight
token shards one after another, each through the C ABI exactly as a rank
would (hyper-parallel "linear_attention_context_parallel.py": the halo of the
K-1 pre-conv rows before the shard, _all_to_all_previous_rank_halo; the final
state of the shard's last sequence handed to the next shard as the initial
state of its first, _SendFinalStateP2PFunction / _RecvInitialStateP2PFunction;
fla "context.py" get_cp_cu_seqlens for the local cu_seqlens and metadata):

  forward   rank r: localise, conv with the halo rows, chunk forward with
            h0[0] = the previous shard's ht when pre_num_ranks > 0;
  backward  ranks in reverse: dht of the last local sequence = the next
            shard's dh0[0] when post_num_ranks > 0, and each shard's dhalo is
            added into the previous shard's last K-1 rows of dx.

The concatenated o, ht, dx, dw, dg, dbeta and dh0 must equal the unsplit GPU
run and the fp64 oracle run end to end on the whole batch."""
import dataclasses

import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn, workloads
from oracle import capi
from tests.helpers import assert_close, cu_tensor, f64, split_qkv

pytestmark = pytest.mark.gpu

WS = 8


def _batch(g_scale):
    spec = workloads.config("shard3of8_32k_h16_d128_bf16")
    # the whole batch: same seed and length rule, no shard split
    full = dataclasses.replace(spec, world_size=1, rank=0, halo=False, g_scale=g_scale)
    inp = workloads.make(full)
    T = inp["T"]
    gen = torch.Generator().manual_seed(7)
    do = (torch.randn(T, spec.Hv, spec.dv, generator=gen)).to(torch.bfloat16)
    dht = torch.randn(inp["cap"], spec.Hv, spec.dk, spec.dv, generator=gen) * 0.01
    return spec, inp, do, dht


def _run_sharded(spec, inp, do, dht):
    Hk, Hv, dk, dv, K = spec.Hk, spec.Hv, spec.dk, spec.dv, spec.K
    cu_glob = inp["cu_global"]
    total = int(cu_glob[-1])
    part = total // WS
    x, w = inp["x"].cuda(), inp["w"].cuda()
    g, beta, h0 = inp["g"].cuda(), inp["beta"].cuda(), inp["h0"].cuda()
    cu_dev = cu_tensor(cu_glob)
    ranks = []
    carry = None  # ht of the previous shard's last local sequence
    o_parts, ht_final = [], torch.zeros_like(h0)
    for r in range(WS):
        local, meta = gdn.gdn_localize_cu_seqlens(cu_dev, total, WS, r, K)
        m = gdn.read_meta(meta)
        n = m["num_local_seqs"]
        first = m["first_seq_global_idx"]
        rs, re = m["rank_start"], m["rank_end"]
        print("  rank %d: [%d, %d) %d local sequences from %d, pre %d post %d n_halo %d"
              % (r, rs, re, n, first, m["pre_num_ranks"], m["post_num_ranks"], m["n_halo"]),
              flush=True)
        lc = local[:n + 1].contiguous()
        halo = x[rs - (K - 1):rs].contiguous() if r > 0 else None
        h0_r = h0[first:first + n].clone()
        if m["pre_num_ranks"] > 0:
            h0_r[0] = carry
        y = gdn.gdn_conv1d_silu_halo(x[rs:re], w, lc, halo=halo, meta=meta if r > 0 else None)
        o, ht = gdn.gdn_chunk_fwd(y, g[rs:re].contiguous(), beta[rs:re].contiguous(), lc, Hk, Hv,
                                  dk, dv, h0=h0_r)
        carry = ht[n - 1].clone()
        o_parts.append(o)
        # a sequence's final state is the one of the shard holding its last token
        for i in range(n):
            gi = first + i
            if i < n - 1 or m["post_num_ranks"] == 0:
                ht_final[gi] = ht[i]
        ranks.append(dict(m=m, lc=lc, halo=halo, meta=meta, y=y, h0=h0_r, rs=rs, re=re))
    # backward, last shard first
    dx = torch.zeros((total, spec.C), dtype=torch.float32, device="cuda")
    dw = torch.zeros((spec.C, K), dtype=torch.float32, device="cuda")
    dg = torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    dh0 = torch.zeros_like(h0)
    back = None  # dh0[0] of the next shard
    dht_d, do_d = dht.cuda(), do.cuda()
    for r in reversed(range(WS)):
        R = ranks[r]
        m, n, first, rs, re = R["m"], R["m"]["num_local_seqs"], R["m"]["first_seq_global_idx"], \
            R["rs"], R["re"]
        dht_r = dht_d[first:first + n].clone()
        if m["post_num_ranks"] > 0:
            dht_r[n - 1] = back
        gr = gdn.gdn_chunk_bwd(R["y"], g[rs:re].contiguous(), beta[rs:re].contiguous(), R["lc"],
                               Hk, Hv, dk, dv, do_d[rs:re].contiguous(), h0=R["h0"], dht=dht_r)
        dx_r, dw_r, _, dhalo = gdn.gdn_conv1d_silu_halo_bwd(
            x[rs:re], w, R["lc"], gr["dy"], halo=R["halo"], meta=R["meta"] if r > 0 else None)
        dx[rs:re] += dx_r.float()
        if dhalo is not None:
            dx[rs - (K - 1):rs] += dhalo.float()
        dw += dw_r
        dg[rs:re] = gr["dg"]
        dbeta[rs:re] = gr["dbeta"]
        back = gr["dh0"][0].clone()
        for i in range(n):
            if i > 0 or m["pre_num_ranks"] == 0:
                dh0[first + i] = gr["dh0"][i]
    torch.cuda.synchronize()
    return dict(o=torch.cat(o_parts), ht=ht_final, dx=dx, dw=dw, dg=dg, dbeta=dbeta, dh0=dh0)


def _run_unsplit(spec, inp, do, dht):
    Hk, Hv, dk, dv = spec.Hk, spec.Hv, spec.dk, spec.dv
    cu = cu_tensor(inp["cu_global"])
    x, w = inp["x"].cuda(), inp["w"].cuda()
    g, beta, h0 = inp["g"].cuda(), inp["beta"].cuda(), inp["h0"].cuda()
    y = gdn.gdn_conv1d_silu_halo(x, w, cu)
    o, ht = gdn.gdn_chunk_fwd(y, g, beta, cu, Hk, Hv, dk, dv, h0=h0)
    gr = gdn.gdn_chunk_bwd(y, g, beta, cu, Hk, Hv, dk, dv, do.cuda(), h0=h0, dht=dht.cuda())
    dx, dw, _, _ = gdn.gdn_conv1d_silu_halo_bwd(x, w, cu, gr["dy"])
    torch.cuda.synchronize()
    return dict(o=o, ht=ht, dx=dx, dw=dw, dg=gr["dg"], dbeta=gr["dbeta"], dh0=gr["dh0"])


def _oracle(spec, inp, do, dht):
    Hk, Hv, d = spec.Hk, spec.Hv, spec.dk
    cu = inp["cu_global"]
    xh, wh = f64(inp["x"]), f64(inp["w"])
    yr = capi.conv1d_silu(xh, wh, None, None, 0, cu)
    q, k, v = split_qkv(yr, Hk, Hv, d, d)
    o, ht = capi.gdn_fwd(q, k, v, f64(inp["g"]), f64(inp["beta"]), f64(inp["h0"]), cu, d ** -0.5)
    e = capi.gdn_bwd(q, k, v, f64(inp["g"]), f64(inp["beta"]), f64(inp["h0"]), cu, d ** -0.5,
                     f64(do), f64(dht))
    T = yr.shape[0]
    dyr = np.concatenate([e["dq"].reshape(T, -1), e["dk"].reshape(T, -1), e["dv"].reshape(T, -1)], 1)
    dx, dw, _, _ = capi.conv1d_silu_bwd(xh, wh, None, None, 0, cu, dyr)
    return dict(o=o, ht=ht, dx=dx, dw=dw, dg=e["dg"], dbeta=e["dbeta"], dh0=e["dh0"])


@pytest.mark.parametrize("g_scale", [0.02, 1.0])
def test_sharded_chain_equals_unsplit(g_scale):
    """Eight shards chained through ht -> h0[0], halo rows, dh0 -> dht and
    dhalo -> dx equal the unsplit batch; with slow decay (g x 0.02) the
    carried states and their gradients matter across every shard boundary."""
    spec, inp, do, dht = _batch(g_scale)
    sh = _run_sharded(spec, inp, do, dht)
    un = _run_unsplit(spec, inp, do, dht)
    dt = torch.bfloat16
    for key in ("o", "ht", "dx", "dw", "dg", "dbeta", "dh0"):
        assert_close(key + "(vs unsplit)", f64(sh[key]), f64(un[key]), dt)
    if g_scale != 1.0:
        ref = _oracle(spec, inp, do, dht)
        for key in ("o", "ht", "dx", "dw", "dg", "dbeta", "dh0"):
            assert_close(key + "(e2e)", f64(sh[key]), ref[key], dt)
