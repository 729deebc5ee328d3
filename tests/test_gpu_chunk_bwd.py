"""GPU reverse mode (gdn_chunk_bwd, gdn_conv1d_silu_halo_bwd) against the
oracle's hand-written reverse mode.

Small cases: ragged tails, empty sequences, GQA head sharing (dq, dk summed
over the value heads of a q/k head), random initial state and final-state
gradient, l2norm on/off, the segmented state pass, and the training pair
gdn_chunk_fwd_save / gdn_chunk_bwd_saved (the forward keeps the per-chunk
states and records, the backward reads them).  Workloads: the float32
single sequence and the 4 x 4096 bfloat16 batch end to end (conv forward,
chunk forward, chunk backward, conv backward) at full size, the latter also
through the saved pair."""

import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn, workloads
from oracle import capi
from tests.helpers import forced_segments, TOL, assert_close, cu_tensor, f64, split_qkv

pytestmark = pytest.mark.gpu


def _inputs(seed, lengths, Hk, Hv, d, dtype, h0=True):
    gen = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    C = 2 * Hk * d + Hv * d
    y = torch.nn.functional.silu(torch.randn(T, C, generator=gen)).to(dtype)
    beta = torch.sigmoid(torch.randn(T, Hv, generator=gen))
    g = -torch.nn.functional.softplus(torch.randn(T, Hv, generator=gen))
    N = len(lengths)
    h = torch.randn(N, Hv, d, d, generator=gen) * 0.05 if h0 else None
    do = torch.randn(T, Hv, d, generator=gen).to(dtype)
    dht = torch.randn(N, Hv, d, d, generator=gen) * 0.01
    cu = [0] + list(np.cumsum(lengths))
    return y, g, beta, h, do, dht, cu


def _check_bwd(y, g, beta, h0, do, dht, cu, Hk, Hv, d, use_l2norm=True, seg=None):
    dtype = y.dtype
    with forced_segments(seg or 0):
        r = gdn.gdn_chunk_bwd(y.cuda(), g.cuda(), beta.cuda(), cu_tensor(cu), Hk, Hv, d, d,
                              do.cuda(), h0=None if h0 is None else h0.cuda(),
                              dht=None if dht is None else dht.cuda(), use_qk_l2norm=use_l2norm)
        torch.cuda.synchronize()
    q, k, v = split_qkv(f64(y), Hk, Hv, d, d)
    ref = capi.gdn_bwd(q, k, v, f64(g), f64(beta), f64(h0), cu, d ** -0.5, f64(do), f64(dht),
                       use_l2norm)
    dq, dk, dv = split_qkv(f64(r["dy"]), Hk, Hv, d, d)
    assert_close("dq", dq, ref["dq"], dtype)
    assert_close("dk", dk, ref["dk"], dtype)
    assert_close("dv", dv, ref["dv"], dtype)
    assert_close("dbeta", f64(r["dbeta"]), ref["dbeta"], dtype)
    assert_close("dg", f64(r["dg"]), ref["dg"], dtype)
    assert_close("dh0", f64(r["dh0"]), ref["dh0"], dtype)
    return r


SMALL = [
    # lengths, Hk, Hv, d, dtype
    ([256], 2, 2, 32, torch.float32),
    ([1, 63, 64, 65, 0, 130], 1, 2, 32, torch.float32),
    ([200, 77], 2, 2, 64, torch.float32),
    ([300], 2, 4, 128, torch.bfloat16),
    ([1, 63, 64, 65, 0, 129, 250], 2, 2, 128, torch.bfloat16),
    ([190, 70], 1, 2, 64, torch.bfloat16),
]


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_small(ci):
    lengths, Hk, Hv, d, dtype = SMALL[ci]
    print("case", SMALL[ci], flush=True)
    y, g, beta, h0, do, dht, cu = _inputs(ci, lengths, Hk, Hv, d, dtype)
    _check_bwd(y, g, beta, h0, do, dht, cu, Hk, Hv, d)


@pytest.mark.parametrize("seg", [1, 3])
def test_segmented_state_pass(seg):
    y, g, beta, h0, do, dht, cu = _inputs(50 + seg, [1, 64, 130, 0, 400], 2, 4, 128, torch.bfloat16)
    _check_bwd(y, g * 0.05, beta, h0, do, dht, cu, 2, 4, 128, seg=seg)


def test_segmented_state_pass_d64():
    """Head size 64 in bfloat16 with segments of 2 chunks: the final dS pass
    from segment inputs, with replay and summaries both taken."""
    y, g, beta, h0, do, dht, cu = _inputs(61, [1, 64, 130, 0, 400], 2, 4, 64, torch.bfloat16)
    g[:, 2:] *= 0.02
    _check_bwd(y, g, beta, h0, do, dht, cu, 2, 4, 64, seg=2)


@pytest.mark.parametrize("variant", ["mixed_heads", "beta_above_one"])
def test_replay_and_summaries(variant):
    """Both recurrences (the forward's states and the backward's dS) choose
    per (sequence, head) between replaying the chunks next to a segment and
    summaries + scan.  Segments of 3 chunks; mixed_heads: value heads 0-1
    decay fast (replay), 2-3 slowly (summaries); beta_above_one: one head's
    write strengths reach 1.5 on some tokens (no bound there).  Against the
    oracle, saved pair included."""
    y, g, beta, h0, do, dht, cu = _inputs(400 + len(variant), [1, 700, 129, 0, 1300], 2, 4, 128,
                                          torch.bfloat16)
    if variant == "mixed_heads":
        g[:, 2:] *= 0.02
    else:
        beta[900:1000, 1] = 1.5
    r = _check_bwd(y, g, beta, h0, do, dht, cu, 2, 4, 128, seg=3)
    yc, gc, bc, h0c = y.cuda(), g.cuda(), beta.cuda(), h0.cuda()
    with forced_segments(3):
        _, _, saved = gdn.gdn_chunk_fwd_save(yc, gc, bc, cu_tensor(cu), 2, 4, 128, 128, h0=h0c)
        r2 = gdn.gdn_chunk_bwd_saved(yc, gc, bc, cu_tensor(cu), 2, 4, 128, 128, do.cuda(), saved,
                                     h0=h0c, dht=dht.cuda())
        torch.cuda.synchronize()
    for key in r:
        assert_close(key + "(saved vs recomputed)", f64(r2[key]), f64(r[key]), torch.bfloat16)


def test_no_l2norm_no_state():
    y, g, beta, _, do, _, cu = _inputs(9, [150, 40], 2, 2, 32, torch.float32, h0=False)
    _check_bwd(y * 0.1, g, beta, None, do, None, cu, 2, 2, 32, use_l2norm=False)


def test_empty_batch_passes_dht_through():
    d = 32
    y = torch.empty(0, 3 * d, device="cuda")
    dht = torch.randn(2, 1, d, d, device="cuda")
    r = gdn.gdn_chunk_bwd(y, torch.empty(0, 1, device="cuda"), torch.empty(0, 1, device="cuda"),
                          cu_tensor([0, 0, 0]), 1, 1, d, d, torch.empty(0, 1, d, device="cuda"),
                          dht=dht)
    assert torch.equal(r["dh0"], dht)


def test_deterministic():
    y, g, beta, h0, do, dht, cu = _inputs(3, [300, 200], 2, 2, 128, torch.bfloat16)
    args = (y.cuda(), g.cuda(), beta.cuda(), cu_tensor(cu), 2, 2, 128, 128, do.cuda())
    r1 = gdn.gdn_chunk_bwd(*args, h0=h0.cuda(), dht=dht.cuda())
    r2 = gdn.gdn_chunk_bwd(*args, h0=h0.cuda(), dht=dht.cuda())
    for key in r1:
        assert torch.equal(r1[key], r2[key]), key


@pytest.mark.parametrize("name", ["single_t256_h2_d32_f32", "fwdbwd_4x4096_h16_d128_bf16"])
def test_workload_forward_backward(name):
    """conv -> chunk forward -> chunk backward -> conv backward on the GPU;
    per stage against the oracle fed the GPU's y, and end to end (dx, dw,
    dhalo, dg, dbeta, dh0) against the oracle in fp64 from x."""
    spec = workloads.config(name)
    inp = workloads.make(spec)
    dtype = workloads.ACT_DTYPES[spec.act]
    Hk, Hv, d = spec.Hk, spec.Hv, spec.dk
    cu = cu_tensor(inp["cu_global"])
    cu_host = inp["cu_global"]
    n_halo = spec.n_halo if inp["halo"] is not None else 0
    meta = gdn.make_meta("cuda", n_halo=n_halo) if n_halo else None
    x, w = inp["x"].cuda(), inp["w"].cuda()
    halo = None if inp["halo"] is None else inp["halo"].cuda()
    h0 = None if inp["h0"] is None else inp["h0"].cuda()
    y = gdn.gdn_conv1d_silu_halo(x, w, cu, halo=halo, meta=meta)
    g, beta = inp["g"].cuda(), inp["beta"].cuda()
    r = gdn.gdn_chunk_bwd(y, g, beta, cu, Hk, Hv, d, d, inp["do"].cuda(), h0=h0,
                          dht=inp["dht"].cuda())
    dx, dw, _, dhalo = gdn.gdn_conv1d_silu_halo_bwd(x, w, cu, r["dy"], halo=halo, meta=meta)
    torch.cuda.synchronize()
    # per stage: the chunk backward from the GPU's y
    q, k, v = split_qkv(f64(y), Hk, Hv, d, d)
    ref = capi.gdn_bwd(q, k, v, f64(inp["g"]), f64(inp["beta"]), f64(inp["h0"]), cu_host,
                       d ** -0.5, f64(inp["do"]), f64(inp["dht"]))
    dq, dk, dv = split_qkv(f64(r["dy"]), Hk, Hv, d, d)
    assert_close("dq", dq, ref["dq"], dtype)
    assert_close("dk", dk, ref["dk"], dtype)
    assert_close("dv", dv, ref["dv"], dtype)
    assert_close("dbeta", f64(r["dbeta"]), ref["dbeta"], dtype)
    assert_close("dg", f64(r["dg"]), ref["dg"], dtype)
    assert_close("dh0", f64(r["dh0"]), ref["dh0"], dtype)
    # end to end from x in fp64
    xh, wh, hh = f64(inp["x"]), f64(inp["w"]), f64(inp["halo"])
    yr = capi.conv1d_silu(xh, wh, None, hh, n_halo, cu_host)
    q, k, v = split_qkv(yr, Hk, Hv, d, d)
    e = capi.gdn_bwd(q, k, v, f64(inp["g"]), f64(inp["beta"]), f64(inp["h0"]), cu_host, d ** -0.5,
                     f64(inp["do"]), f64(inp["dht"]))
    T = yr.shape[0]
    dyr = np.concatenate([e["dq"].reshape(T, -1), e["dk"].reshape(T, -1), e["dv"].reshape(T, -1)], 1)
    rdx, rdw, _, rdh = capi.conv1d_silu_bwd(xh, wh, None, hh, n_halo, cu_host, dyr)
    assert_close("dx(e2e)", f64(dx), rdx, dtype)
    assert_close("dw(e2e)", f64(dw), rdw, dtype)
    if dhalo is not None:
        assert_close("dhalo(e2e)", f64(dhalo), rdh, dtype)
    assert_close("dg(e2e)", f64(r["dg"]), e["dg"], dtype)
    assert_close("dbeta(e2e)", f64(r["dbeta"]), e["dbeta"], dtype)
    assert_close("dh0(e2e)", f64(r["dh0"]), e["dh0"], dtype)


SAVED = [
    # lengths, Hk, Hv, d, dtype, forced segment chunks (0: the plan's own)
    ([256], 2, 2, 32, torch.float32, 0),
    ([1, 63, 64, 65, 0, 130], 1, 2, 64, torch.float32, 0),
    ([300, 0, 77], 2, 4, 128, torch.bfloat16, 0),
    ([1, 63, 64, 65, 0, 129, 250], 2, 2, 128, torch.bfloat16, 2),
    ([190, 70], 1, 2, 64, torch.bfloat16, 0),
    ([3000], 1, 1, 128, torch.bfloat16, 0),  # one sequence: the forward's first-segment plan
]


@pytest.mark.parametrize("ci", range(len(SAVED)))
def test_saved_pair(ci):
    """gdn_chunk_fwd_save returns gdn_chunk_fwd's o and ht bit for bit;
    gdn_chunk_bwd_saved from its buffer matches the oracle and agrees with
    gdn_chunk_bwd (which recomputes the forward) to the dtype's bar."""
    lengths, Hk, Hv, d, dtype, seg = SAVED[ci]
    print("case", SAVED[ci], flush=True)
    y, g, beta, h0, do, dht, cu = _inputs(200 + ci, lengths, Hk, Hv, d, dtype)
    yc, gc, bc, h0c = y.cuda(), g.cuda(), beta.cuda(), h0.cuda()
    cut = cu_tensor(cu)
    with forced_segments(seg):
        o1, ht1 = gdn.gdn_chunk_fwd(yc, gc, bc, cut, Hk, Hv, d, d, h0=h0c)
        o2, ht2, saved = gdn.gdn_chunk_fwd_save(yc, gc, bc, cut, Hk, Hv, d, d, h0=h0c)
        r1 = gdn.gdn_chunk_bwd(yc, gc, bc, cut, Hk, Hv, d, d, do.cuda(), h0=h0c, dht=dht.cuda())
        r2 = gdn.gdn_chunk_bwd_saved(yc, gc, bc, cut, Hk, Hv, d, d, do.cuda(), saved, h0=h0c,
                                     dht=dht.cuda())
        torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    q, k, v = split_qkv(f64(y), Hk, Hv, d, d)
    ref = capi.gdn_bwd(q, k, v, f64(g), f64(beta), f64(h0), cu, d ** -0.5, f64(do), f64(dht), True)
    dq, dk, dv = split_qkv(f64(r2["dy"]), Hk, Hv, d, d)
    assert_close("dq", dq, ref["dq"], dtype)
    assert_close("dk", dk, ref["dk"], dtype)
    assert_close("dv", dv, ref["dv"], dtype)
    assert_close("dbeta", f64(r2["dbeta"]), ref["dbeta"], dtype)
    assert_close("dg", f64(r2["dg"]), ref["dg"], dtype)
    assert_close("dh0", f64(r2["dh0"]), ref["dh0"], dtype)
    for key in r1:
        assert_close(key + "(vs recomputed)", f64(r2[key]), f64(r1[key]), dtype)


def test_saved_pair_workload():
    """The 4 x 4096 bfloat16 batch through the saved pair: the backward from
    the forward's buffer against the oracle and the recomputing backward."""
    spec = workloads.config("fwdbwd_4x4096_h16_d128_bf16")
    inp = workloads.make(spec)
    Hk, Hv, d = spec.Hk, spec.Hv, spec.dk
    cu = cu_tensor(inp["cu_global"])
    meta = gdn.make_meta("cuda", n_halo=spec.n_halo)
    y = gdn.gdn_conv1d_silu_halo(inp["x"].cuda(), inp["w"].cuda(), cu, halo=inp["halo"].cuda(),
                                 meta=meta)
    g, beta, h0 = inp["g"].cuda(), inp["beta"].cuda(), inp["h0"].cuda()
    do, dht = inp["do"].cuda(), inp["dht"].cuda()
    _, _, saved = gdn.gdn_chunk_fwd_save(y, g, beta, cu, Hk, Hv, d, d, h0=h0)
    r2 = gdn.gdn_chunk_bwd_saved(y, g, beta, cu, Hk, Hv, d, d, do, saved, h0=h0, dht=dht)
    r1 = gdn.gdn_chunk_bwd(y, g, beta, cu, Hk, Hv, d, d, do, h0=h0, dht=dht)
    torch.cuda.synchronize()
    q, k, v = split_qkv(f64(y), Hk, Hv, d, d)
    ref = capi.gdn_bwd(q, k, v, f64(inp["g"]), f64(inp["beta"]), f64(inp["h0"]),
                       inp["cu_global"], d ** -0.5, f64(inp["do"]), f64(inp["dht"]))
    dq, dk, dv = split_qkv(f64(r2["dy"]), Hk, Hv, d, d)
    assert_close("dq", dq, ref["dq"], torch.bfloat16)
    assert_close("dk", dk, ref["dk"], torch.bfloat16)
    assert_close("dv", dv, ref["dv"], torch.bfloat16)
    assert_close("dbeta", f64(r2["dbeta"]), ref["dbeta"], torch.bfloat16)
    assert_close("dg", f64(r2["dg"]), ref["dg"], torch.bfloat16)
    assert_close("dh0", f64(r2["dh0"]), ref["dh0"], torch.bfloat16)
    for key in r1:
        assert_close(key + "(vs recomputed)", f64(r2[key]), f64(r1[key]), torch.bfloat16)
