"""Thin Python binding of libgdn's C ABI (include/gdn.h).

Argument marshalling only: every entry point takes torch tensors that already
live on the GPU, checks dtypes/shapes/contiguity, and passes raw device
pointers plus the current HIP stream to the library.  All arithmetic happens
in the HIP kernels; there is no fallback.  Loading fails loudly when the
in-tree ``libgdn.so`` is missing (build it with
``python -m linear_attention_sequence_causal_amd.build``).

Function names match the C entry points.
"""
from __future__ import annotations

import ctypes
import os
import struct
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EHIP, GDN_EWORKSPACE = 0, -1, -2, -3, -4
GDN_F32, GDN_BF16 = 0, 1
META_OK, META_NOT_MONOTONE, META_BAD_TOTAL = 0, 1, 2

# gdn_cp_meta: 3 x int64 then 8 x int32 (56 bytes)
META_FORMAT = "<qqqiiiiiiii"
META_FIELDS = ("rank_start", "rank_end", "pre_num_conv_tokens", "num_local_seqs",
               "first_seq_global_idx", "is_first_rank", "is_last_rank", "pre_num_ranks",
               "post_num_ranks", "n_halo", "status")
META_BYTES = struct.calcsize(META_FORMAT)

ENTRY_POINTS = (
    "gdn_localize_cu_seqlens", "gdn_conv1d_silu_halo", "gdn_conv_bwd_workspace_size",
    "gdn_conv1d_silu_halo_bwd", "gdn_chunk_workspace_size", "gdn_chunk_fwd", "gdn_chunk_bwd",
    "gdn_last_error",
)


class GdnError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s failed (status %d): %s" % (fn, code, msg))
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libgdn.so and declares the C signatures (no GPU needed)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libgdn.so not found at %s; build it with "
                           "`python -m linear_attention_sequence_causal_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    INT = ctypes.c_int
    lib.gdn_localize_cu_seqlens.argtypes = [P, I32, I64, I32, I32, I32, P, P, P]
    lib.gdn_conv1d_silu_halo.argtypes = [P, P, P, P, P, I32, I64, I32, I32, P, P, INT, P]
    lib.gdn_conv_bwd_workspace_size.argtypes = [I64, I32, I32]
    lib.gdn_conv_bwd_workspace_size.restype = SZ
    lib.gdn_conv1d_silu_halo_bwd.argtypes = [P, P, P, P, P, I32, I64, I32, I32, P, P, P, P, P, P,
                                             P, SZ, INT, P]
    lib.gdn_chunk_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, INT, INT]
    lib.gdn_chunk_workspace_size.restype = SZ
    lib.gdn_chunk_fwd.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32, F,
                                  INT, P, P, P, SZ, INT, P]
    lib.gdn_chunk_bwd.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32, F,
                                  INT, P, P, P, P, I64, P, I64, P, P, P, P, SZ, INT, P]
    lib.gdn_last_error.restype = ctypes.c_char_p
    for name in ENTRY_POINTS:
        if name not in ("gdn_conv_bwd_workspace_size", "gdn_chunk_workspace_size", "gdn_last_error"):
            getattr(lib, name).restype = INT
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(fn: str, rc: int):
    if rc != GDN_OK:
        raise GdnError(fn, rc, _lib.gdn_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError("activations must be bfloat16 or float32, got %s" % t.dtype)


def _req(t, name, dtype=None, dev=None, contiguous=True):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _ws(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# metadata
# --------------------------------------------------------------------------
def make_meta(device, n_halo: int = 0, **fields) -> torch.Tensor:
    """A gdn_cp_meta built on the host (e.g. a halo without a shard split)."""
    vals = dict.fromkeys(META_FIELDS, 0)
    vals.update(fields)
    vals["n_halo"] = n_halo
    raw = struct.pack(META_FORMAT, *(int(vals[f]) for f in META_FIELDS))
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(device)


def read_meta(meta: torch.Tensor) -> dict:
    raw = bytes(meta.cpu().numpy().tobytes())
    return dict(zip(META_FIELDS, struct.unpack(META_FORMAT, raw)))


def gdn_localize_cu_seqlens(cu_seqlens: torch.Tensor, total_tokens: int, world_size: int,
                            rank: int, conv_kernel_size: int, out=None):
    """Returns (local_cu_seqlens int32 [num_seqs+1], meta uint8[56]) on the
    device of cu_seqlens; no host synchronisation.  ``out`` may supply both
    buffers."""
    load_library()
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    n = cu_seqlens.numel() - 1
    if out is not None:
        local, meta = out
        _req(local, "local_cu_seqlens", torch.int32)
        if local.numel() < n + 1 or meta.numel() < META_BYTES:
            raise ValueError("output buffers too small")
    else:
        local = torch.empty(n + 1, dtype=torch.int32, device=cu_seqlens.device)
        meta = torch.empty(META_BYTES, dtype=torch.uint8, device=cu_seqlens.device)
    rc = _lib.gdn_localize_cu_seqlens(_ptr(cu_seqlens), n, int(total_tokens), world_size, rank,
                                      conv_kernel_size, _ptr(local), _ptr(meta), _stream())
    _check("gdn_localize_cu_seqlens", rc)
    return local, meta


# --------------------------------------------------------------------------
# conv
# --------------------------------------------------------------------------
def gdn_conv1d_silu_halo(x, w, cu_seqlens, bias=None, halo=None, meta=None, out=None):
    """y [T, C] = SiLU(causal depthwise conv(x)) with the halo rows of meta."""
    load_library()
    T, C = x.shape
    K = w.shape[1]
    for t, nm in ((x, "x"), (w, "w"), (bias, "bias"), (halo, "halo")):
        _req(t, nm, x.dtype)
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    y = torch.empty_like(x) if out is None else out
    rc = _lib.gdn_conv1d_silu_halo(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), _ptr(cu_seqlens),
                                   cu_seqlens.numel() - 1, T, C, K, _ptr(meta), _ptr(y), _dt(x),
                                   _stream())
    _check("gdn_conv1d_silu_halo", rc)
    return y


def gdn_conv1d_silu_halo_bwd(x, w, cu_seqlens, dy, bias=None, halo=None, meta=None):
    """Returns dx [T,C] (act), dw [C,K] fp32, dbias [C] fp32 (or None),
    dhalo [K-1,C] (act, or None)."""
    load_library()
    T, C = x.shape
    K = w.shape[1]
    for t, nm in ((x, "x"), (w, "w"), (bias, "bias"), (halo, "halo"), (dy, "dy")):
        _req(t, nm, x.dtype)
    dx = torch.empty_like(x)
    dw = torch.empty((C, K), dtype=torch.float32, device=x.device)
    dbias = torch.empty(C, dtype=torch.float32, device=x.device) if bias is not None else None
    dhalo = torch.empty((K - 1, C), dtype=x.dtype, device=x.device) if halo is not None else None
    nbytes = _lib.gdn_conv_bwd_workspace_size(T, C, K)
    ws = _ws(nbytes, x.device)
    rc = _lib.gdn_conv1d_silu_halo_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), _ptr(cu_seqlens),
                                       cu_seqlens.numel() - 1, T, C, K, _ptr(meta), _ptr(dy),
                                       _ptr(dx), _ptr(dw), _ptr(dbias), _ptr(dhalo), _ptr(ws),
                                       nbytes, _dt(x), _stream())
    _check("gdn_conv1d_silu_halo_bwd", rc)
    return dx, dw, dbias, dhalo


# --------------------------------------------------------------------------
# chunked gated delta rule
# --------------------------------------------------------------------------
def _qkv_views(y, Hk, Hv, dk, dv):
    """q, k, v views into a conv output y [T, C] (channels [Q | K | V])."""
    T, C = y.shape
    if C != 2 * Hk * dk + Hv * dv:
        raise ValueError("C=%d does not match 2*Hk*dk + Hv*dv" % C)
    return y[:, :Hk * dk], y[:, Hk * dk:2 * Hk * dk], y[:, 2 * Hk * dk:]


def chunk_workspace_size(T, N, Hk, Hv, dk, dv, dtype, bwd=False) -> int:
    load_library()
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(_lib.gdn_chunk_workspace_size(T, N, Hk, Hv, dk, dv, dt, int(bwd)))


def gdn_chunk_fwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0=None, scale=None,
                  use_qk_l2norm=True, want_ht=True, out=None, ht_out=None, ws=None):
    """Chunked gated delta rule on the q/k/v channel blocks of y [T, C].

    Returns (o [T, Hv, dv] act, ht [N, Hv, dk, dv] fp32 or None)."""
    load_library()
    T, C = y.shape
    N = cu_seqlens.numel() - 1
    _req(y, "y")
    _req(g, "g", torch.float32)
    _req(beta, "beta", torch.float32)
    _req(h0, "h0", torch.float32)
    _req(cu_seqlens, "cu_seqlens", torch.int32)
    if g.shape != (T, Hv) or beta.shape != (T, Hv):
        raise ValueError("g and beta must be [T, Hv]")
    if h0 is not None and h0.shape != (N, Hv, dk, dv):
        raise ValueError("h0 must be [N, Hv, dk, dv]")
    q, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    o = out if out is not None else torch.empty((T, Hv, dv), dtype=y.dtype, device=y.device)
    ht = None
    if want_ht:
        ht = ht_out if ht_out is not None else torch.empty((N, Hv, dk, dv), dtype=torch.float32,
                                                           device=y.device)
    nbytes = chunk_workspace_size(T, N, Hk, Hv, dk, dv, y.dtype)
    if ws is None or ws.numel() < nbytes:
        ws = _ws(nbytes, y.device)
    scale = dk ** -0.5 if scale is None else scale
    rc = _lib.gdn_chunk_fwd(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(h0),
                            _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv, float(scale),
                            int(bool(use_qk_l2norm)), _ptr(o), _ptr(ht), _ptr(ws), nbytes,
                            _dt(y), _stream())
    _check("gdn_chunk_fwd", rc)
    return o, ht


def gdn_chunk_bwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, h0=None, dht=None, scale=None,
                  use_qk_l2norm=True, ws=None):
    """Reverse mode of gdn_chunk_fwd.  Returns dict with dy [T, C] (act: the
    gradients w.r.t. the q, k, v channel blocks of y), dg, dbeta [T, Hv] fp32
    and dh0 [N, Hv, dk, dv] fp32."""
    load_library()
    T, C = y.shape
    N = cu_seqlens.numel() - 1
    _req(y, "y")
    _req(d_o, "d_o", y.dtype)
    _req(dht, "dht", torch.float32)
    _req(h0, "h0", torch.float32)
    q, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    dy = torch.empty_like(y)
    dq, dk_, dv_ = _qkv_views(dy, Hk, Hv, dk, dv)
    dg = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
    dbeta = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
    dh0 = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=y.device)
    nbytes = chunk_workspace_size(T, N, Hk, Hv, dk, dv, y.dtype, bwd=True)
    if ws is None or ws.numel() < nbytes:
        ws = _ws(nbytes, y.device)
    scale = dk ** -0.5 if scale is None else scale
    rc = _lib.gdn_chunk_bwd(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(h0),
                            _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv, float(scale),
                            int(bool(use_qk_l2norm)), _ptr(d_o), _ptr(dht), _ptr(dq), _ptr(dk_), C,
                            _ptr(dv_), C, _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(ws), nbytes,
                            _dt(y), _stream())
    _check("gdn_chunk_bwd", rc)
    return dict(dy=dy, dg=dg, dbeta=dbeta, dh0=dh0)
