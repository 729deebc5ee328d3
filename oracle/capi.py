"""ctypes front end of the fp64 C oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The product library never loads it.

``build()`` compiles ``gdn_oracle.c`` with gcc (-O3, OpenMP) into
``libgdn_oracle.so`` next to the source.  Arrays are converted to contiguous
fp64 (int64 for cu_seqlens) before every call, so callers may pass any
numpy-compatible input.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

META_FIELDS = (
    "rank_start", "rank_end", "num_local_seqs", "first_seq_global_idx",
    "is_first_rank", "is_last_rank", "pre_num_ranks", "post_num_ranks",
    "pre_num_conv_tokens", "n_halo",
)


def build(force: bool = True) -> str:
    """Compile the oracle shared library; returns its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_localize.argtypes = [P, I64, I64, I64, I64, P, P]
        lib.oracle_localize.restype = ctypes.c_int
        lib.oracle_conv1d_silu.argtypes = [P, P, P, P, I64, P, I64, I64, I64, I64, P, P]
        lib.oracle_conv1d_silu.restype = None
        lib.oracle_conv1d_silu_bwd.argtypes = [P, P, P, P, I64, P, I64, I64, I64, I64, P, P, P, P, P]
        lib.oracle_conv1d_silu_bwd.restype = None
        lib.oracle_gdn_fwd.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                       ctypes.c_double, ctypes.c_int, P, P, ctypes.c_int]
        lib.oracle_gdn_fwd.restype = None
        lib.oracle_gdn_bwd.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                       ctypes.c_double, ctypes.c_int, P, P, P, P, P, P, P, P,
                                       ctypes.c_int]
        lib.oracle_gdn_bwd.restype = None
        lib.oracle_gating_fwd.argtypes = [P, P, I64, P, P, I64, I64, P, P]
        lib.oracle_gating_fwd.restype = None
        lib.oracle_gating_bwd.argtypes = [P, P, I64, P, P, P, P, I64, I64, P, P, I64, P, P]
        lib.oracle_gating_bwd.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def localize(cu, world_size, rank, conv_k):
    """Returns (local_cu int64, meta dict) or raises ValueError."""
    lib = _load()
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    n = len(cu) - 1
    local = np.zeros(n + 1, dtype=np.int64)
    meta = np.zeros(len(META_FIELDS), dtype=np.int64)
    rc = lib.oracle_localize(_ptr(cu), n, world_size, rank, conv_k, _ptr(local), _ptr(meta))
    if rc != 0:
        raise ValueError("localisation undefined for these arguments")
    m = dict(zip(META_FIELDS, (int(x) for x in meta)))
    return local[: m["num_local_seqs"] + 1].copy(), m


def conv1d_silu(x, w, bias, halo, n_halo, cu, return_z=False):
    lib = _load()
    x, w, bias, halo = _f64(x), _f64(w), _f64(bias), _f64(halo)
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    T, C = x.shape
    K = w.shape[1]
    y = np.zeros((T, C))
    z = np.zeros((T, C)) if return_z else None
    lib.oracle_conv1d_silu(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), int(n_halo), _ptr(cu),
                           len(cu) - 1, T, C, K, _ptr(y), _ptr(z))
    return (y, z) if return_z else y


def conv1d_silu_bwd(x, w, bias, halo, n_halo, cu, dy):
    """Returns dx [T,C], dw [C,K], dbias [C] (or None), dhalo [K-1,C] (or None)."""
    lib = _load()
    x, w, bias, halo, dy = _f64(x), _f64(w), _f64(bias), _f64(halo), _f64(dy)
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    T, C = x.shape
    K = w.shape[1]
    dx = np.zeros((T, C))
    dw = np.zeros((C, K))
    dbias = np.zeros(C) if bias is not None else None
    dhalo = np.zeros((max(K - 1, 0), C)) if halo is not None else None
    lib.oracle_conv1d_silu_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), int(n_halo), _ptr(cu),
                               len(cu) - 1, T, C, K, _ptr(dy), _ptr(dx), _ptr(dw), _ptr(dbias),
                               _ptr(dhalo))
    return dx, dw, dbias, dhalo


def gdn_fwd(q, k, v, g, beta, h0, cu, scale, use_l2norm=True, nthreads=None):
    """q,k [T,Hk,dk]; v [T,Hv,dv]; g,beta [T,Hv]; h0 [N,Hv,dk,dv] or None.
    Returns o [T,Hv,dv], ht [N,Hv,dk,dv]."""
    lib = _load()
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    ht = np.zeros((N, Hv, dk, dv))
    nt = nthreads if nthreads else max_threads()
    lib.oracle_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu), N, T,
                       Hk, Hv, dk, dv, float(scale), int(bool(use_l2norm)), _ptr(o), _ptr(ht), nt)
    return o, ht


def gdn_bwd(q, k, v, g, beta, h0, cu, scale, do, dht, use_l2norm=True, nthreads=None):
    """Returns dict dq, dk [T,Hk,dk], dv [T,Hv,dv], dg, dbeta [T,Hv],
    dh0 [N,Hv,dk,dv] -- gradients w.r.t. the raw (pre-l2norm) q, k."""
    lib = _load()
    q, k, v, g, beta, h0, do, dht = map(_f64, (q, k, v, g, beta, h0, do, dht))
    cu = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    N = len(cu) - 1
    out = dict(dq=np.zeros((T, Hk, dk)), dk=np.zeros((T, Hk, dk)), dv=np.zeros((T, Hv, dv)),
               dg=np.zeros((T, Hv)), dbeta=np.zeros((T, Hv)), dh0=np.zeros((N, Hv, dk, dv)))
    nt = nthreads if nthreads else max_threads()
    lib.oracle_gdn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu), N, T,
                       Hk, Hv, dk, dv, float(scale), int(bool(use_l2norm)), _ptr(do), _ptr(dht),
                       _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                       _ptr(out["dbeta"]), _ptr(out["dh0"]), nt)
    return out


def gating_fwd(a, b, A_log, dt_bias):
    """a, b [T, Hv]; A_log, dt_bias [Hv].  Returns g, beta [T, Hv]:
    beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias)."""
    lib = _load()
    a, b, A_log, dt_bias = map(_f64, (a, b, A_log, dt_bias))
    T, Hv = a.shape
    g, beta = np.zeros((T, Hv)), np.zeros((T, Hv))
    lib.oracle_gating_fwd(_ptr(a), _ptr(b), Hv, _ptr(A_log), _ptr(dt_bias), T, Hv, _ptr(g),
                          _ptr(beta))
    return g, beta


def gating_bwd(a, b, A_log, dt_bias, dg, dbeta):
    """Reverse mode of gating_fwd: returns dict da, db [T, Hv], dA_log,
    ddt_bias [Hv]."""
    lib = _load()
    a, b, A_log, dt_bias, dg, dbeta = map(_f64, (a, b, A_log, dt_bias, dg, dbeta))
    T, Hv = a.shape
    out = dict(da=np.zeros((T, Hv)), db=np.zeros((T, Hv)), dA_log=np.zeros(Hv),
               ddt_bias=np.zeros(Hv))
    lib.oracle_gating_bwd(_ptr(a), _ptr(b), Hv, _ptr(A_log), _ptr(dt_bias), _ptr(dg), _ptr(dbeta),
                          T, Hv, _ptr(out["da"]), _ptr(out["db"]), Hv, _ptr(out["dA_log"]),
                          _ptr(out["ddt_bias"]))
    return out
