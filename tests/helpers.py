"""Shared helpers of the GPU parity tests: running the HIP path and the fp64
oracle on the same seeded inputs, and the relative-error metric
max|got - ref| / max|ref| used by every floating-point comparison."""
from __future__ import annotations

import contextlib
import ctypes
import json
import os

import numpy as np
import torch

from linear_attention_sequence_causal_amd import gdn
from oracle import capi

# tolerances of the parity bar: max|d| / max|ref| per output tensor
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref, block=4096) -> float:
    """max|got - ref| / max|ref| (max|got| when ref is all zero), taken over
    blocks of leading rows so that large tensors need little extra memory."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.ndim == 0:
        got, ref = got.reshape(1), ref.reshape(1)
    dmax = rmax = gmax = 0.0
    for r0 in range(0, got.shape[0], block):
        g = np.asarray(got[r0:r0 + block], dtype=np.float64)
        r = np.asarray(ref[r0:r0 + block], dtype=np.float64)
        if g.size == 0:
            continue
        dmax = max(dmax, float(np.abs(g - r).max()))
        rmax = max(rmax, float(np.abs(r).max()))
        gmax = max(gmax, float(np.abs(g).max()))
    return gmax if rmax == 0 else dmax / rmax


def all_finite(a, block=4096) -> bool:
    a = np.asarray(a)
    if a.ndim == 0:
        return bool(np.isfinite(a))
    return all(np.isfinite(np.asarray(a[r0:r0 + block], dtype=np.float64)).all()
               for r0 in range(0, a.shape[0], block))


def log_parity(name, err, tol):
    """Appends one comparison (test id, tensor, max|d|/max|ref|, tolerance)
    as a JSON line to the file named by GDN_PARITY_LOG, when that is set."""
    path = os.environ.get("GDN_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    with open(path, "a") as fh:
        fh.write(json.dumps({"test": test, "tensor": name, "rel_err": float(err),
                             "tol": float(tol)}) + "\n")


def assert_close(name, got, ref, dtype):
    e = rel_err(got, ref)
    print("  %-10s rel err %.3e (tol %.0e)" % (name, e, TOL[dtype]), flush=True)
    log_parity(name, e, TOL[dtype])
    assert all_finite(got), name + " has non-finite values"
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


@contextlib.contextmanager
def forced_segments(chunks):
    """Chunk plans made on this thread cut every sequence into segments of
    ``chunks`` 64-token chunks (the library's test hook, absent from its
    public header)."""
    lib = gdn.load_library()
    fn = lib.gdn_testing_set_segment_chunks
    fn.argtypes = [ctypes.c_int]
    fn.restype = ctypes.c_int
    prev = fn(int(chunks))
    try:
        yield
    finally:
        fn(prev)
