"""Shared helpers of the GPU parity tests: running the HIP path and the fp64
oracle on the same seeded inputs, and the relative-error metric
max|got - ref| / max|ref| used by every floating-point comparison."""
from __future__ import annotations

import numpy as np
import torch

from linear_attention_sequence_causal_amd import gdn
from oracle import capi

# tolerances of the parity bar: max|d| / max|ref| per output tensor
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    print("  %-10s rel err %.3e (tol %.0e)" % (name, e, TOL[dtype]), flush=True)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), name + " has non-finite values"
    assert e <= TOL[dtype], "%s: rel err %.3e > %.0e" % (name, e, TOL[dtype])


def split_qkv(y, Hk, Hv, dk, dv):
    T = y.shape[0]
    q = y[:, :Hk * dk].reshape(T, Hk, dk)
    k = y[:, Hk * dk:2 * Hk * dk].reshape(T, Hk, dk)
    v = y[:, 2 * Hk * dk:].reshape(T, Hv, dv)
    return q, k, v


def oracle_chunk_fwd(y, g, beta, h0, cu, Hk, Hv, dk, dv, scale, heads=None, use_l2norm=True):
    """Oracle forward from a (rounded) y; ``heads`` restricts to a subset of
    value heads (their q/k heads are taken along)."""
    q, k, v = split_qkv(f64(y), Hk, Hv, dk, dv)
    gg, bb, hh = f64(g), f64(beta), f64(h0)
    if heads is None:
        return capi.gdn_fwd(q, k, v, gg, bb, hh, cu, scale, use_l2norm)
    grp = Hv // Hk
    outs = []
    for h in heads:
        a = h // grp
        o, ht = capi.gdn_fwd(q[:, a:a + 1], k[:, a:a + 1], v[:, h:h + 1], gg[:, h:h + 1],
                             bb[:, h:h + 1], None if hh is None else hh[:, h:h + 1], cu, scale,
                             use_l2norm)
        outs.append((o[:, 0], ht[:, 0]))
    return np.stack([o for o, _ in outs], 1), np.stack([h for _, h in outs], 1)


def to_dev(t, device="cuda"):
    return None if t is None else t.to(device)


def cu_tensor(cu, device="cuda"):
    return torch.tensor(np.asarray(cu), dtype=torch.int32, device=device)
