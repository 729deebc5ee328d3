"""gdn_conv1d_silu_halo_bwd_noalloc (the conv backward with the library's
static scratch, for callers that cannot allocate) against the workspace
entry point gdn_conv1d_silu_halo_bwd: two calls in a row through the C ABI,
the second on a smaller input, and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from linear_attention_sequence_causal_amd import gdn
from tests.helpers import assert_close, cu_tensor, f64

pytestmark = pytest.mark.gpu


def _case(seed, lengths, C, K, dtype, with_halo, with_bias):
    gen = torch.Generator().manual_seed(seed)
    T = sum(lengths)
    x = torch.randn(T, C, generator=gen).to(dtype).cuda()
    w = (torch.randn(C, K, generator=gen) / np.sqrt(K)).to(dtype).cuda()
    bias = torch.randn(C, generator=gen).to(dtype).cuda() if with_bias else None
    halo = torch.randn(K - 1, C, generator=gen).to(dtype).cuda() if with_halo else None
    dy = torch.randn(T, C, generator=gen).to(dtype).cuda()
    cu = cu_tensor([0] + list(np.cumsum(lengths)))
    meta = gdn.make_meta("cuda", n_halo=K - 1) if with_halo else None
    return x, w, bias, halo, dy, cu, meta


def _outs(x, w, bias, halo):
    T, C = x.shape
    K = w.shape[1]
    # NaN-filled outputs: every element must be written by the call
    dx = torch.full_like(x, float("nan"))
    dw = torch.full((C, K), float("nan"), device="cuda")
    db = torch.full((C,), float("nan"), device="cuda") if bias is not None else None
    dh = torch.full_like(halo, float("nan")) if halo is not None else None
    return dx, dw, db, dh


CASES = [
    # the second call is smaller than the first
    ([(4096, 3000, 1), 6144, 4, torch.bfloat16, True, True],
     [(700, 0, 65), 2048, 4, torch.bfloat16, True, False]),
    ([(16384,), 8192, 4, torch.bfloat16, False, False],
     [(300, 200), 96, 3, torch.float32, True, True]),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_noalloc_matches_workspace_entry(ci):
    for step, args in enumerate(CASES[ci]):
        lengths, C, K, dtype, with_halo, with_bias = args
        print("case %d call %d: lengths=%s C=%d K=%d %s" % (ci, step, lengths, C, K, dtype),
              flush=True)
        x, w, bias, halo, dy, cu, meta = _case(10 * ci + step, list(lengths), C, K, dtype,
                                               with_halo, with_bias)
        ref = gdn.gdn_conv1d_silu_halo_bwd(x, w, cu, dy, bias=bias, halo=halo, meta=meta)
        got = gdn.gdn_conv1d_silu_halo_bwd_noalloc(x, w, cu, dy, _outs(x, w, bias, halo),
                                                   bias=bias, halo=halo, meta=meta)
        torch.cuda.synchronize()
        for name, g, r in zip(("dx", "dw", "dbias", "dhalo"), got, ref):
            if r is None:
                assert g is None
                continue
            # same kernels, same split of the tokens: identical results
            assert_close(name, f64(g), f64(r), dtype)
            assert torch.equal(g, r), name


def test_noalloc_rejects_inputs_beyond_its_scratch():
    lib = gdn.load_library()
    T, C, K = 1 << 20, 16384, 4
    assert lib.gdn_conv_bwd_workspace_size(T, C, K) > gdn.CONV_BWD_SCRATCH_BYTES
    f = ctypes.c_void_p(0x1000)
    rc = lib.gdn_conv1d_silu_halo_bwd_noalloc(f, f, None, None, f, 1, T, C, K, None, f, f, f,
                                              None, None, 1, None)
    assert rc == gdn.GDN_EWORKSPACE
    assert b"scratch" in lib.gdn_last_error()
