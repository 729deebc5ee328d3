"""GPU gating step (gdn_gating_fwd / gdn_gating_bwd) and the chunk forward
with the gating fused into its kernels (gdn_chunk_fwd_gated), against the
oracle (hyper-parallel "linear_attention_context_parallel.py", the CP
wrappers' beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias)).

The gates are float32 computed from exactly representable inputs, so they
are held to the float32 bar (1e-4) whatever the activation dtype; da, db are
stored in the activation dtype and take its bar."""
import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn, workloads
from oracle import capi
from tests.helpers import assert_close, cu_tensor, f64, oracle_chunk_fwd

pytestmark = pytest.mark.gpu


def _params(seed, Hv):
    rng = np.random.default_rng(seed)
    A_log = torch.tensor(rng.uniform(0.0, np.log(16.0), Hv), dtype=torch.float32)
    dt_bias = torch.tensor(rng.standard_normal(Hv), dtype=torch.float32)
    return A_log, dt_bias


def _packed_ab(seed, T, Hv, dtype, pad):
    """a, b as two column blocks of packed rows [T, 2 Hv + pad] (the layout
    of the page's packed projections), plus contiguous copies."""
    gen = torch.Generator().manual_seed(seed)
    rows = (torch.randn(T, 2 * Hv + pad, generator=gen) * 2).to(dtype)
    return rows, rows[:, :Hv], rows[:, Hv:2 * Hv]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,Hv,pad", [(1, 1, 0), (257, 16, 6), (4096, 32, 0), (0, 4, 2)])
def test_gating_fwd_bwd(dtype, T, Hv, pad):
    rows, a, b = _packed_ab(T + Hv, T, Hv, dtype, pad)
    A_log, dt_bias = _params(T, Hv)
    ra = rows.cuda()
    ad, bd = ra[:, :Hv], ra[:, Hv:2 * Hv]
    g, beta = gdn.gdn_gating_fwd(ad, bd, A_log.cuda(), dt_bias.cuda())
    gen = torch.Generator().manual_seed(3)
    dg = torch.randn(T, Hv, generator=gen)
    dbeta = torch.randn(T, Hv, generator=gen)
    r1 = gdn.gdn_gating_bwd(ad, bd, A_log.cuda(), dt_bias.cuda(), dg.cuda(), dbeta.cuda())
    r2 = gdn.gdn_gating_bwd(ad, bd, A_log.cuda(), dt_bias.cuda(), dg.cuda(), dbeta.cuda())
    torch.cuda.synchronize()
    if T == 0:
        assert g.shape == (0, Hv)
        assert torch.all(r1["dA_log"] == 0) and torch.all(r1["ddt_bias"] == 0)
        return
    rg, rbeta = capi.gating_fwd(f64(a), f64(b), f64(A_log), f64(dt_bias))
    assert_close("g", f64(g), rg, torch.float32)
    assert_close("beta", f64(beta), rbeta, torch.float32)
    ref = capi.gating_bwd(f64(a), f64(b), f64(A_log), f64(dt_bias), f64(dg), f64(dbeta))
    assert_close("da", f64(r1["da"]), ref["da"], dtype)
    assert_close("db", f64(r1["db"]), ref["db"], dtype)
    assert_close("dA_log", f64(r1["dA_log"]), ref["dA_log"], torch.float32)
    assert_close("ddt_bias", f64(r1["ddt_bias"]), ref["ddt_bias"], torch.float32)
    for key in r1:  # fixed-order reductions
        assert torch.equal(r1[key], r2[key]), key


def _gated_case(seed, lengths, Hk, Hv, d, dtype, pad=2):
    gen = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    C = 2 * Hk * d + Hv * d
    y = torch.nn.functional.silu(torch.randn(T, C, generator=gen)).to(dtype)
    h0 = torch.randn(len(lengths), Hv, d, d, generator=gen) * 0.05
    rows, a, b = _packed_ab(seed, T, Hv, dtype, pad)
    A_log, dt_bias = _params(seed, Hv)
    # weaker decay so that the states carry across chunks and segments
    A_log = A_log - 3.0
    cu = [0] + list(np.cumsum(lengths))
    return y, rows, a, b, A_log, dt_bias, h0, cu


@pytest.mark.parametrize("case", [
    ([1, 63, 64, 65, 0, 300], 1, 2, 32, torch.float32),
    ([200, 77], 2, 2, 64, torch.float32),
    ([1, 129, 700, 0, 2600], 2, 4, 128, torch.bfloat16),
    ([190, 65], 2, 2, 64, torch.bfloat16),
])
def test_gated_chunk_fwd(case):
    """Gates formed inside the chunk kernels: identical to gdn_gating_fwd
    followed by gdn_chunk_fwd, and equal to the oracle's gating + recurrence."""
    lengths, Hk, Hv, d, dtype = case
    print("case", case, flush=True)
    y, rows, a, b, A_log, dt_bias, h0, cu = _gated_case(sum(lengths), lengths, Hk, Hv, d, dtype)
    yc, rc = y.cuda(), rows.cuda()
    ad, bd = rc[:, :Hv], rc[:, Hv:2 * Hv]
    cut = cu_tensor(cu)
    o, ht, g_out, b_out = gdn.gdn_chunk_fwd_gated(yc, ad, bd, A_log.cuda(), dt_bias.cuda(), cut,
                                                  Hk, Hv, d, d, h0=h0.cuda(), want_gates=True)
    g, beta = gdn.gdn_gating_fwd(ad, bd, A_log.cuda(), dt_bias.cuda())
    o2, ht2 = gdn.gdn_chunk_fwd(yc, g, beta, cut, Hk, Hv, d, d, h0=h0.cuda())
    torch.cuda.synchronize()
    assert torch.equal(g_out, g) and torch.equal(b_out, beta)
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    rg, rb = capi.gating_fwd(f64(a), f64(b), f64(A_log), f64(dt_bias))
    ro, rht = oracle_chunk_fwd(y, torch.tensor(rg), torch.tensor(rb), h0, cu, Hk, Hv, d, d,
                               d ** -0.5)
    assert_close("o", f64(o), ro, dtype)
    assert_close("ht", f64(ht), rht, dtype)


def test_gated_long_workload():
    """The 131072-token, 16/32-head workload with its gates formed from
    bfloat16 projections inside the chunk kernels, every head against the
    oracle's gating and recurrence (fp64), and against the unfused path."""
    spec = workloads.config("long131k_hk16_hv32_d128_bf16")
    inp = workloads.make(spec)
    Hk, Hv, d = spec.Hk, spec.Hv, spec.dk
    T = inp["T"]
    cu = cu_tensor(inp["cu_global"])
    y = gdn.gdn_conv1d_silu_halo(inp["x"].cuda(), inp["w"].cuda(), cu)
    gen = torch.Generator().manual_seed(11)
    ab = torch.randn(T, 2 * Hv, generator=gen).to(torch.bfloat16).cuda()
    ad, bd = ab[:, :Hv], ab[:, Hv:]
    A_log, dt_bias = _params(11, Hv)
    A_log = A_log - 4.0  # slow decay: states carry over the segments
    o, ht, g, beta = gdn.gdn_chunk_fwd_gated(y, ad, bd, A_log.cuda(), dt_bias.cuda(), cu, Hk, Hv, d,
                                             d, want_gates=True)
    o2, ht2 = gdn.gdn_chunk_fwd(y, g, beta, cu, Hk, Hv, d, d)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ht, ht2)
    rg, rb = capi.gating_fwd(f64(ad), f64(bd), f64(A_log), f64(dt_bias))
    assert_close("g", f64(g), rg, torch.float32)
    assert_close("beta", f64(beta), rb, torch.float32)
    ro, rht = oracle_chunk_fwd(y.cpu(), torch.tensor(rg), torch.tensor(rb), None,
                               inp["cu_global"], Hk, Hv, d, d, d ** -0.5)
    assert_close("o", f64(o), ro, torch.bfloat16)
    assert_close("ht", f64(ht), rht, torch.bfloat16)
