"""GPU head-sharded (Ulysses) entry gdn_ulysses_fwd against the oracle and
against the unsplit model.

hyper-parallel "linear_attention_context_parallel.py",
LinearAttentionUlyssesCPWrapper: _seq_to_head_qkvba packs, per rank r, the
columns [q_r | k_r | v_r | b_r | a_r] of its heads (q_r, k_r: key-dim slice r,
v_r: value-dim slice r, b_r, a_r: v-head slice r); _local_conv_weight takes
the matching rows of the conv weight; A_log and dt_bias are sliced by v-head.
Run rank by rank on one GPU, the ranks' outputs, put side by side on the head
dimension, must equal the model run unsplit."""
import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn, workloads
from oracle import capi
from tests.helpers import assert_close, cu_tensor, f64, split_qkv

pytestmark = pytest.mark.gpu


def _pack_rank(x, ab, Hk, Hv, dk, dv, cp, r, pad=0):
    """The page's packing for rank r of cp: x [T, 2 Hk dk + Hv dv] holds the
    model's [q | k | v] projections, ab [T, 2 Hv] its [b | a]."""
    lk, lv, lh = Hk * dk // cp, Hv * dv // cp, Hv // cp
    kd = Hk * dk
    cols = [x[:, r * lk:(r + 1) * lk], x[:, kd + r * lk:kd + (r + 1) * lk],
            x[:, 2 * kd + r * lv:2 * kd + (r + 1) * lv], ab[:, r * lh:(r + 1) * lh],
            ab[:, Hv + r * lh:Hv + (r + 1) * lh]]
    if pad:
        cols.append(torch.zeros(x.shape[0], pad, dtype=x.dtype, device=x.device))
    return torch.cat(cols, dim=1).contiguous()


def _local_rows(w, Hk, Hv, dk, dv, cp, r):
    """Rows of a per-channel parameter (conv weight or bias) for rank r."""
    lk, lv = Hk * dk // cp, Hv * dv // cp
    kd = Hk * dk
    idx = torch.cat([torch.arange(r * lk, (r + 1) * lk), torch.arange(kd + r * lk, kd + (r + 1) * lk),
                     torch.arange(2 * kd + r * lv, 2 * kd + (r + 1) * lv)])
    return w[idx.to(w.device)].contiguous()


def _oracle_rank(x, w, bias, ab, A_log, dt_bias, cu, Hk, Hv, dk, dv, cp, r):
    """conv over the rank's channels, gating, recurrence: fp64, from x."""
    lh = Hv // cp
    xs = _local_rows(x.t(), Hk, Hv, dk, dv, cp, r).t()
    ws = _local_rows(w, Hk, Hv, dk, dv, cp, r)
    bs = None if bias is None else _local_rows(bias, Hk, Hv, dk, dv, cp, r)
    yr = capi.conv1d_silu(f64(xs), f64(ws), f64(bs), None, 0, cu)
    g, beta = capi.gating_fwd(f64(ab[:, Hv + r * lh:Hv + (r + 1) * lh]),
                              f64(ab[:, r * lh:(r + 1) * lh]), f64(A_log[r * lh:(r + 1) * lh]),
                              f64(dt_bias[r * lh:(r + 1) * lh]))
    q, k, v = split_qkv(yr, Hk // cp, lh, dk, dv)
    return yr, capi.gdn_fwd(q, k, v, g, beta, None, cu, dk ** -0.5)


def _params(seed, Hv, C, K, dtype, with_bias):
    gen = torch.Generator().manual_seed(seed)
    A_log = torch.rand(Hv, generator=gen) * np.log(16.0) - 4.0
    dt_bias = torch.randn(Hv, generator=gen)
    w = (torch.randn(C, K, generator=gen) / np.sqrt(K)).to(dtype)
    bias = torch.randn(C, generator=gen).to(dtype) if with_bias else None
    return A_log, dt_bias, w, bias


def _run_ranks(x, ab, w, bias, A_log, dt_bias, cu, Hk, Hv, dk, dv, cp, pad=0):
    outs, ys = [], []
    for r in range(cp):
        packed = _pack_rank(x, ab, Hk, Hv, dk, dv, cp, r, pad)
        lh = Hv // cp
        y, o, _, _, _ = gdn.gdn_ulysses_fwd(
            packed, _local_rows(w, Hk, Hv, dk, dv, cp, r), A_log[r * lh:(r + 1) * lh].contiguous(),
            dt_bias[r * lh:(r + 1) * lh].contiguous(), cu, Hk // cp, Hv // cp, dk, dv,
            conv_bias=None if bias is None else _local_rows(bias, Hk, Hv, dk, dv, cp, r))
        outs.append(o)
        ys.append(y)
    return torch.cat(outs, dim=1), ys


SMALL = [
    # lengths, Hk, Hv, d, cp, dtype, bias, pad
    ([300, 0, 77], 2, 4, 32, 2, torch.float32, True, 0),
    ([1, 63, 64, 65, 200], 2, 2, 32, 2, torch.float32, False, 3),   # scalar conv path
    ([700, 129], 4, 8, 128, 4, torch.bfloat16, True, 0),
    ([500], 2, 4, 64, 2, torch.bfloat16, False, 5),                # unaligned rows
]


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_ulysses_small(ci):
    lengths, Hk, Hv, d, cp, dtype, with_bias, pad = SMALL[ci]
    print("case", SMALL[ci], flush=True)
    T = sum(lengths)
    C = 2 * Hk * d + Hv * d
    gen = torch.Generator().manual_seed(ci)
    x = torch.randn(T, C, generator=gen).to(dtype)
    ab = torch.randn(T, 2 * Hv, generator=gen).to(dtype)
    A_log, dt_bias, w, bias = _params(ci, Hv, C, 4, dtype, with_bias)
    cu = [0] + list(np.cumsum(lengths))
    xd, abd = x.cuda(), ab.cuda()
    bd = None if bias is None else bias.cuda()
    o, ys = _run_ranks(xd, abd, w.cuda(), bd, A_log.cuda(), dt_bias.cuda(), cu_tensor(cu), Hk, Hv,
                       d, d, cp, pad)
    torch.cuda.synchronize()
    for r in range(cp):
        yr, (ro, _) = _oracle_rank(x, w, bias, ab, A_log, dt_bias, cu, Hk, Hv, d, d, cp, r)
        lh = Hv // cp
        assert_close("y[%d]" % r, f64(ys[r]), yr, dtype)
        assert_close("o[%d]" % r, f64(o[:, r * lh:(r + 1) * lh]), ro, dtype)


def test_ulysses_long_workload_eight_ranks():
    """The 131072-token model (16 q/k, 32 v heads, d = 128) as 8 Ulysses
    ranks of 2 q/k and 4 v heads each: the ranks side by side equal the
    unsplit conv + gated chunk forward, and rank 3 equals the oracle."""
    spec = workloads.config("long131k_hk16_hv32_d128_bf16")
    inp = workloads.make(spec)
    Hk, Hv, d, cp = spec.Hk, spec.Hv, spec.dk, 8
    T = inp["T"]
    gen = torch.Generator().manual_seed(21)
    ab = torch.randn(T, 2 * Hv, generator=gen).to(torch.bfloat16)
    A_log, dt_bias, _, _ = _params(21, Hv, spec.C, spec.K, torch.bfloat16, False)
    x, w = inp["x"].cuda(), inp["w"].cuda()
    abd, Ad, dbd = ab.cuda(), A_log.cuda(), dt_bias.cuda()
    cu = cu_tensor(inp["cu_global"])
    o, ys = _run_ranks(x, abd, w, None, Ad, dbd, cu, Hk, Hv, d, d, cp)
    y = gdn.gdn_conv1d_silu_halo(x, w, cu)
    o_full, _, _, _ = gdn.gdn_chunk_fwd_gated(y, abd[:, Hv:], abd[:, :Hv], Ad, dbd, cu, Hk, Hv, d,
                                              d, want_ht=False)
    torch.cuda.synchronize()
    assert_close("o(vs unsplit)", f64(o), f64(o_full), torch.bfloat16)
    r = 3
    yr, (ro, _) = _oracle_rank(inp["x"], inp["w"], None, ab, A_log, dt_bias, inp["cu_global"], Hk,
                               Hv, d, d, cp, r)
    lh = Hv // cp
    assert_close("y[3]", f64(ys[r]), yr, torch.bfloat16)
    assert_close("o[3]", f64(o[:, r * lh:(r + 1) * lh]), ro, torch.bfloat16)
