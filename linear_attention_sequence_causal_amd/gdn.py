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
    "gdn_chunk_summary_workspace_size", "gdn_chunk_summary", "gdn_merge_summaries",
    "gdn_conv1d_silu_halo_bwd_noalloc", "gdn_gating_fwd", "gdn_gating_bwd_workspace_size",
    "gdn_gating_bwd", "gdn_chunk_fwd_gated_workspace_size", "gdn_chunk_fwd_gated",
    "gdn_ulysses_fwd_workspace_size", "gdn_ulysses_fwd", "gdn_chunk_saved_size",
    "gdn_chunk_fwd_save", "gdn_chunk_bwd_saved", "gdn_last_error",
)
CONV_BWD_SCRATCH_BYTES = 16 << 20  # GDN_CONV_BWD_SCRATCH_BYTES
_SIZE_QUERIES = ("gdn_conv_bwd_workspace_size", "gdn_chunk_workspace_size",
                 "gdn_chunk_summary_workspace_size", "gdn_gating_bwd_workspace_size",
                 "gdn_chunk_fwd_gated_workspace_size", "gdn_ulysses_fwd_workspace_size",
                 "gdn_chunk_saved_size")


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
    lib.gdn_conv1d_silu_halo_bwd_noalloc.argtypes = [P, P, P, P, P, I32, I64, I32, I32, P, P, P,
                                                     P, P, P, INT, P]
    lib.gdn_chunk_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, INT, INT]
    lib.gdn_chunk_workspace_size.restype = SZ
    lib.gdn_chunk_fwd.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32, F,
                                  INT, P, P, P, SZ, INT, P]
    lib.gdn_chunk_bwd.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32, F,
                                  INT, P, P, P, P, I64, P, I64, P, P, P, P, SZ, INT, P]
    lib.gdn_chunk_saved_size.argtypes = [I64, I32, I32, I32, I32, I32, INT]
    lib.gdn_chunk_saved_size.restype = SZ
    lib.gdn_chunk_fwd_save.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32,
                                       F, INT, P, P, P, SZ, P, SZ, INT, P]
    lib.gdn_chunk_bwd_saved.argtypes = [P, P, I64, P, I64, P, P, P, P, I32, I64, I32, I32, I32, I32,
                                        F, INT, P, P, P, P, I64, P, I64, P, P, P, P, SZ, P, SZ,
                                        INT, P]
    lib.gdn_chunk_summary_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, INT]
    lib.gdn_chunk_summary_workspace_size.restype = SZ
    lib.gdn_chunk_summary.argtypes = [P, I64, P, I64, P, P, P, I32, I64, I32, I32, I32, I32, INT,
                                      P, P, P, SZ, INT, P]
    lib.gdn_merge_summaries.argtypes = [P, P, I32, I32, I32, I32, P, P, P]
    lib.gdn_gating_fwd.argtypes = [P, P, I64, P, P, I64, I32, P, P, INT, P]
    lib.gdn_gating_bwd_workspace_size.argtypes = [I64, I32]
    lib.gdn_gating_bwd_workspace_size.restype = SZ
    lib.gdn_gating_bwd.argtypes = [P, P, I64, P, P, P, P, I64, I32, P, P, I64, P, P, P, SZ, INT, P]
    lib.gdn_chunk_fwd_gated_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, INT]
    lib.gdn_chunk_fwd_gated_workspace_size.restype = SZ
    lib.gdn_chunk_fwd_gated.argtypes = [P, P, I64, P, I64, P, P, I64, P, P, P, P, I32, I64, I32,
                                        I32, I32, I32, F, INT, P, P, P, P, P, SZ, INT, P]
    lib.gdn_ulysses_fwd_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, INT]
    lib.gdn_ulysses_fwd_workspace_size.restype = SZ
    lib.gdn_ulysses_fwd.argtypes = [P, I64, P, P, I32, P, P, P, P, I32, I64, I32, I32, I32, I32, F,
                                    INT, P, P, P, P, P, P, SZ, INT, P]
    lib.gdn_last_error.restype = ctypes.c_char_p
    for name in ENTRY_POINTS:
        if name not in _SIZE_QUERIES + ("gdn_last_error",):
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


def _req(t, name, dtype=None, shape=None, contiguous=True, device=None):
    """Checks a tensor argument (None passes): on the GPU, of ``dtype``, of
    ``shape`` (a tuple, None entries free) and contiguous; ``device`` (a
    tensor) must hold it on the same device."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device.device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device.device))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None:
        ok = t.dim() == len(shape) and all(w is None or int(w) == d for w, d in zip(shape, t.shape))
        if not ok:
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if contiguous and not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _workspace(ws, nbytes: int, like: torch.Tensor) -> Optional[torch.Tensor]:
    """The caller's workspace if it is large enough (uint8, contiguous, on
    the device of ``like``), else a new one; None when none is needed."""
    if nbytes == 0:
        return None
    if ws is not None:
        _req(ws, "ws", torch.uint8, (None,), device=like)
        if ws.numel() >= nbytes:
            return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


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
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,))
    n = cu_seqlens.numel() - 1
    if out is not None:
        local, meta = out
        _req(local, "local_cu_seqlens", torch.int32, (None,), device=cu_seqlens)
        _req(meta, "meta", torch.uint8, (None,), device=cu_seqlens)
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
    _req(x, "x", shape=(None, None))
    T, C = x.shape
    _req(w, "w", x.dtype, (C, None), device=x)
    K = w.shape[1]
    _req(bias, "bias", x.dtype, (C,), device=x)
    _req(halo, "halo", x.dtype, (K - 1, C), device=x)
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=x)
    _req(meta, "meta", torch.uint8, (META_BYTES,), device=x)
    _req(out, "out", x.dtype, (T, C), device=x)
    y = torch.empty_like(x) if out is None else out
    rc = _lib.gdn_conv1d_silu_halo(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), _ptr(cu_seqlens),
                                   cu_seqlens.numel() - 1, T, C, K, _ptr(meta), _ptr(y), _dt(x),
                                   _stream())
    _check("gdn_conv1d_silu_halo", rc)
    return y


def conv_bwd_workspace_size(T, C, K) -> int:
    load_library()
    return int(_lib.gdn_conv_bwd_workspace_size(T, C, K))


def gdn_conv1d_silu_halo_bwd(x, w, cu_seqlens, dy, bias=None, halo=None, meta=None, out=None,
                             ws=None):
    """Returns dx [T,C] (act), dw [C,K] fp32, dbias [C] fp32 (or None),
    dhalo [K-1,C] (act, or None).  ``out`` may supply (dx, dw, dbias, dhalo)
    and ``ws`` the workspace, so that the call allocates nothing."""
    load_library()
    _req(x, "x", shape=(None, None))
    T, C = x.shape
    _req(w, "w", x.dtype, (C, None), device=x)
    K = w.shape[1]
    _req(bias, "bias", x.dtype, (C,), device=x)
    _req(halo, "halo", x.dtype, (K - 1, C), device=x)
    _req(dy, "dy", x.dtype, (T, C), device=x)
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=x)
    _req(meta, "meta", torch.uint8, (META_BYTES,), device=x)
    if out is not None:
        dx, dw, dbias, dhalo = out
        if (dbias is None) != (bias is None) or (dhalo is None) != (halo is None):
            raise ValueError("out must hold dbias / dhalo exactly when bias / halo are given")
    else:
        dx = torch.empty_like(x)
        dw = torch.empty((C, K), dtype=torch.float32, device=x.device)
        dbias = torch.empty(C, dtype=torch.float32, device=x.device) if bias is not None else None
        dhalo = torch.empty((K - 1, C), dtype=x.dtype, device=x.device) if halo is not None else None
    _req(dx, "dx", x.dtype, (T, C), device=x)
    _req(dw, "dw", torch.float32, (C, K), device=x)
    _req(dbias, "dbias", torch.float32, (C,), device=x)
    _req(dhalo, "dhalo", x.dtype, (K - 1, C), device=x)
    nbytes = conv_bwd_workspace_size(T, C, K)
    ws = _workspace(ws, nbytes, x)
    rc = _lib.gdn_conv1d_silu_halo_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), _ptr(cu_seqlens),
                                       cu_seqlens.numel() - 1, T, C, K, _ptr(meta), _ptr(dy),
                                       _ptr(dx), _ptr(dw), _ptr(dbias), _ptr(dhalo), _ptr(ws),
                                       nbytes, _dt(x), _stream())
    _check("gdn_conv1d_silu_halo_bwd", rc)
    return dx, dw, dbias, dhalo


def gdn_conv1d_silu_halo_bwd_noalloc(x, w, cu_seqlens, dy, out, bias=None, halo=None,
                                     meta=None):
    """gdn_conv1d_silu_halo_bwd into the caller's ``out`` = (dx, dw, dbias,
    dhalo) with the library's static scratch: neither this function nor the
    library allocates device memory."""
    load_library()
    _req(x, "x", shape=(None, None))
    T, C = x.shape
    _req(w, "w", x.dtype, (C, None), device=x)
    K = w.shape[1]
    _req(bias, "bias", x.dtype, (C,), device=x)
    _req(halo, "halo", x.dtype, (K - 1, C), device=x)
    _req(dy, "dy", x.dtype, (T, C), device=x)
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=x)
    _req(meta, "meta", torch.uint8, (META_BYTES,), device=x)
    dx, dw, dbias, dhalo = out
    if (dbias is None) != (bias is None) or (dhalo is None) != (halo is None):
        raise ValueError("out must hold dbias / dhalo exactly when bias / halo are given")
    _req(dx, "dx", x.dtype, (T, C), device=x)
    _req(dw, "dw", torch.float32, (C, K), device=x)
    _req(dbias, "dbias", torch.float32, (C,), device=x)
    _req(dhalo, "dhalo", x.dtype, (K - 1, C), device=x)
    rc = _lib.gdn_conv1d_silu_halo_bwd_noalloc(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo),
                                               _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, C, K,
                                               _ptr(meta), _ptr(dy), _ptr(dx), _ptr(dw),
                                               _ptr(dbias), _ptr(dhalo), _dt(x), _stream())
    _check("gdn_conv1d_silu_halo_bwd_noalloc", rc)
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


def _chunk_common(y, g, beta, cu_seqlens, h0, Hk, Hv, dk, dv):
    _req(y, "y", shape=(None, None))
    T = y.shape[0]
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=y)
    N = cu_seqlens.numel() - 1
    _req(g, "g", torch.float32, (T, Hv), device=y)
    _req(beta, "beta", torch.float32, (T, Hv), device=y)
    _req(h0, "h0", torch.float32, (N, Hv, dk, dv), device=y)
    return T, N


def chunk_saved_size(T, N, Hk, Hv, dk, dv, dtype) -> int:
    load_library()
    dt = GDN_BF16 if dtype == torch.bfloat16 else GDN_F32
    return int(_lib.gdn_chunk_saved_size(T, N, Hk, Hv, dk, dv, dt))


def gdn_chunk_fwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0=None, scale=None,
                  use_qk_l2norm=True, want_ht=True, out=None, ht_out=None, ws=None):
    """Chunked gated delta rule on the q/k/v channel blocks of y [T, C].

    Returns (o [T, Hv, dv] act, ht [N, Hv, dk, dv] fp32 or None)."""
    o, ht, _ = _chunk_fwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0, scale, use_qk_l2norm,
                          want_ht, out, ht_out, ws, None, False)
    return o, ht


def gdn_chunk_fwd_save(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0=None, scale=None,
                       use_qk_l2norm=True, want_ht=True, out=None, ht_out=None, ws=None,
                       saved=None):
    """gdn_chunk_fwd that also fills ``saved`` (uint8, chunk_saved_size
    bytes; allocated when None) for gdn_chunk_bwd_saved.  Returns (o, ht,
    saved)."""
    return _chunk_fwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0, scale, use_qk_l2norm, want_ht,
                      out, ht_out, ws, saved, True)


def _chunk_fwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, h0, scale, use_qk_l2norm, want_ht, out,
               ht_out, ws, saved, save):
    load_library()
    T, N = _chunk_common(y, g, beta, cu_seqlens, h0, Hk, Hv, dk, dv)
    C = y.shape[1]
    q, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    _req(out, "out", y.dtype, (T, Hv, dv), device=y)
    _req(ht_out, "ht_out", torch.float32, (N, Hv, dk, dv), device=y)
    o = out if out is not None else torch.empty((T, Hv, dv), dtype=y.dtype, device=y.device)
    ht = None
    if want_ht:
        ht = ht_out if ht_out is not None else torch.empty((N, Hv, dk, dv), dtype=torch.float32,
                                                           device=y.device)
    nbytes = chunk_workspace_size(T, N, Hk, Hv, dk, dv, y.dtype)
    ws = _workspace(ws, nbytes, y)
    scale = dk ** -0.5 if scale is None else scale
    if not save:
        rc = _lib.gdn_chunk_fwd(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(h0),
                                _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv, float(scale),
                                int(bool(use_qk_l2norm)), _ptr(o), _ptr(ht), _ptr(ws), nbytes,
                                _dt(y), _stream())
        _check("gdn_chunk_fwd", rc)
        return o, ht, None
    sbytes = chunk_saved_size(T, N, Hk, Hv, dk, dv, y.dtype)
    saved = _saved_buffer(saved, sbytes, y)
    rc = _lib.gdn_chunk_fwd_save(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(h0),
                                 _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv, float(scale),
                                 int(bool(use_qk_l2norm)), _ptr(o), _ptr(ht), _ptr(saved),
                                 saved.numel(), _ptr(ws), nbytes, _dt(y), _stream())
    _check("gdn_chunk_fwd_save", rc)
    return o, ht, saved


def _saved_buffer(saved, nbytes, like):
    """The saved-state buffer: the caller's (uint8, on like's device, at
    least nbytes) or a new one."""
    if saved is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
    _req(saved, "saved", torch.uint8, (None,), device=like)
    if saved.numel() < nbytes:
        raise ValueError("saved buffer holds %d bytes, needs %d" % (saved.numel(), nbytes))
    return saved


def gdn_chunk_bwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, h0=None, dht=None, scale=None,
                  use_qk_l2norm=True, ws=None, out=None):
    """Reverse mode of gdn_chunk_fwd.  Returns dict with dy [T, C] (act: the
    gradients w.r.t. the q, k, v channel blocks of y), dg, dbeta [T, Hv] fp32
    and dh0 [N, Hv, dk, dv] fp32.  ``out`` may supply (dy, dg, dbeta, dh0)
    and ``ws`` the workspace, so that the call allocates nothing."""
    return _chunk_bwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, h0, dht, scale, use_qk_l2norm,
                      ws, out, None)


def gdn_chunk_bwd_saved(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, saved, h0=None, dht=None,
                        scale=None, use_qk_l2norm=True, ws=None, out=None):
    """gdn_chunk_bwd from the buffer of gdn_chunk_fwd_save on the same inputs."""
    if saved is None:
        raise ValueError("gdn_chunk_bwd_saved needs the saved buffer")
    return _chunk_bwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, h0, dht, scale, use_qk_l2norm,
                      ws, out, saved)


def _chunk_bwd(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, d_o, h0, dht, scale, use_qk_l2norm, ws,
               out, saved):
    load_library()
    T, N = _chunk_common(y, g, beta, cu_seqlens, h0, Hk, Hv, dk, dv)
    C = y.shape[1]
    _req(d_o, "d_o", y.dtype, (T, Hv, dv), device=y)
    _req(dht, "dht", torch.float32, (N, Hv, dk, dv), device=y)
    q, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    if out is not None:
        dy, dg, dbeta, dh0 = out
    else:
        dy = torch.empty_like(y)
        dg = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
        dbeta = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
        dh0 = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=y.device)
    _req(dy, "dy", y.dtype, (T, C), device=y)
    _req(dg, "dg", torch.float32, (T, Hv), device=y)
    _req(dbeta, "dbeta", torch.float32, (T, Hv), device=y)
    _req(dh0, "dh0", torch.float32, (N, Hv, dk, dv), device=y)
    dq, dk_, dv_ = _qkv_views(dy, Hk, Hv, dk, dv)
    nbytes = chunk_workspace_size(T, N, Hk, Hv, dk, dv, y.dtype, bwd=True)
    ws = _workspace(ws, nbytes, y)
    scale = dk ** -0.5 if scale is None else scale
    if saved is None:
        rc = _lib.gdn_chunk_bwd(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(h0),
                                _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv, float(scale),
                                int(bool(use_qk_l2norm)), _ptr(d_o), _ptr(dht), _ptr(dq),
                                _ptr(dk_), C, _ptr(dv_), C, _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                _ptr(ws), nbytes, _dt(y), _stream())
        _check("gdn_chunk_bwd", rc)
    else:
        sbytes = chunk_saved_size(T, N, Hk, Hv, dk, dv, y.dtype)
        saved = _saved_buffer(saved, sbytes, y)
        rc = _lib.gdn_chunk_bwd_saved(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta),
                                      _ptr(h0), _ptr(cu_seqlens), N, T, Hk, Hv, dk, dv,
                                      float(scale), int(bool(use_qk_l2norm)), _ptr(d_o),
                                      _ptr(dht), _ptr(dq), _ptr(dk_), C, _ptr(dv_), C, _ptr(dg),
                                      _ptr(dbeta), _ptr(dh0), _ptr(saved), saved.numel(),
                                      _ptr(ws), nbytes, _dt(y), _stream())
        _check("gdn_chunk_bwd_saved", rc)
    return dict(dy=dy, dg=dg, dbeta=dbeta, dh0=dh0)


# --------------------------------------------------------------------------
# affine state summaries (a shard's [M | E]) and their prefix merge
# --------------------------------------------------------------------------
def gdn_chunk_summary(y, g, beta, cu_seqlens, Hk, Hv, dk, dv, use_qk_l2norm=True, want_m=True,
                      want_e=True, ws=None):
    """Per local sequence n and value head h: S_out = M S_in + E.  Returns
    (M [N, Hv, dk, dk] fp32 or None, E [N, Hv, dk, dv] fp32 or None)."""
    load_library()
    T, N = _chunk_common(y, g, beta, cu_seqlens, None, Hk, Hv, dk, dv)
    C = y.shape[1]
    _, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    M = torch.empty((N, Hv, dk, dk), dtype=torch.float32, device=y.device) if want_m else None
    E = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=y.device) if want_e else None
    dt = GDN_BF16 if y.dtype == torch.bfloat16 else GDN_F32
    nbytes = int(_lib.gdn_chunk_summary_workspace_size(T, N, Hk, Hv, dk, dv, dt))
    ws = _workspace(ws, nbytes, y)
    rc = _lib.gdn_chunk_summary(_ptr(k), C, _ptr(v), C, _ptr(g), _ptr(beta), _ptr(cu_seqlens), N,
                                T, Hk, Hv, dk, dv, int(bool(use_qk_l2norm)), _ptr(M), _ptr(E),
                                _ptr(ws), nbytes, _dt(y), _stream())
    _check("gdn_chunk_summary", rc)
    return M, E


def gdn_merge_summaries(M, E, h_in=None, out=None):
    """M [R, ..., dk, dk], E [R, ..., dk, dv] (the same middle dimensions, the
    state slots); h = h_in (or zero), then h <- M[r] h + E[r] for r < R.
    Returns h [..., dk, dv] fp32."""
    load_library()
    _req(M, "M", torch.float32)
    if M.dim() < 3:
        raise ValueError("M must be [R, ..., dk, dk]")
    R, dk = M.shape[0], M.shape[-1]
    slots = tuple(M.shape[1:-2])
    _req(M, "M", torch.float32, (R,) + slots + (dk, dk))
    _req(E, "E", torch.float32, (R,) + slots + (dk, None), device=M)
    dv = E.shape[-1]
    _req(h_in, "h_in", torch.float32, slots + (dk, dv), device=M)
    h = out if out is not None else torch.empty(slots + (dk, dv), dtype=torch.float32,
                                                device=M.device)
    _req(h, "out", torch.float32, slots + (dk, dv), device=M)
    S = 1
    for d in slots:
        S *= int(d)
    rc = _lib.gdn_merge_summaries(_ptr(M), _ptr(E), R, S, dk, dv, _ptr(h_in), _ptr(h), _stream())
    _check("gdn_merge_summaries", rc)
    return h


# --------------------------------------------------------------------------
# gating: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias)
# --------------------------------------------------------------------------
def _ab_views(a, b, Hv):
    """a, b [T, Hv] views that share one token stride (columns of packed
    rows or contiguous tensors); returns (T, ld)."""
    if a.dim() != 2 or b.shape != a.shape or a.shape[1] != Hv:
        raise ValueError("a and b must be [T, Hv] views of one shape")
    if a.stride(1) != 1 or b.stride(1) != 1 or a.stride(0) != b.stride(0):
        raise ValueError("a and b need unit head stride and one common token stride")
    if a.dtype != b.dtype or a.device != b.device or not a.is_cuda:
        raise ValueError("a and b must be GPU tensors of one dtype")
    return a.shape[0], a.stride(0)


def gdn_gating_fwd(a, b, A_log, dt_bias, out=None):
    """Returns (g, beta) float32 [T, Hv]."""
    load_library()
    Hv = A_log.numel()
    T, ld = _ab_views(a, b, Hv)
    _req(A_log, "A_log", torch.float32, (Hv,), device=a)
    _req(dt_bias, "dt_bias", torch.float32, (Hv,), device=a)
    g, beta = out if out is not None else (
        torch.empty((T, Hv), dtype=torch.float32, device=a.device),
        torch.empty((T, Hv), dtype=torch.float32, device=a.device))
    _req(g, "g", torch.float32, (T, Hv), device=a)
    _req(beta, "beta", torch.float32, (T, Hv), device=a)
    rc = _lib.gdn_gating_fwd(_ptr(a), _ptr(b), ld, _ptr(A_log), _ptr(dt_bias), T, Hv, _ptr(g),
                             _ptr(beta), _dt(a), _stream())
    _check("gdn_gating_fwd", rc)
    return g, beta


def gdn_gating_bwd(a, b, A_log, dt_bias, dg, dbeta, ws=None):
    """Returns dict da, db [T, Hv] (activations), dA_log, ddt_bias [Hv]."""
    load_library()
    Hv = A_log.numel()
    T, ld = _ab_views(a, b, Hv)
    _req(A_log, "A_log", torch.float32, (Hv,), device=a)
    _req(dt_bias, "dt_bias", torch.float32, (Hv,), device=a)
    _req(dg, "dg", torch.float32, (T, Hv), device=a)
    _req(dbeta, "dbeta", torch.float32, (T, Hv), device=a)
    da = torch.empty((T, Hv), dtype=a.dtype, device=a.device)
    db = torch.empty((T, Hv), dtype=a.dtype, device=a.device)
    dA = torch.empty(Hv, dtype=torch.float32, device=a.device)
    ddt = torch.empty(Hv, dtype=torch.float32, device=a.device)
    nbytes = int(_lib.gdn_gating_bwd_workspace_size(T, Hv))
    ws = _workspace(ws, nbytes, a)
    rc = _lib.gdn_gating_bwd(_ptr(a), _ptr(b), ld, _ptr(A_log), _ptr(dt_bias), _ptr(dg),
                             _ptr(dbeta), T, Hv, _ptr(da), _ptr(db), Hv, _ptr(dA), _ptr(ddt),
                             _ptr(ws), nbytes, _dt(a), _stream())
    _check("gdn_gating_bwd", rc)
    return dict(da=da, db=db, dA_log=dA, ddt_bias=ddt)


def gdn_chunk_fwd_gated(y, a, b, A_log, dt_bias, cu_seqlens, Hk, Hv, dk, dv, h0=None,
                        scale=None, use_qk_l2norm=True, want_ht=True, want_gates=False, out=None,
                        ws=None):
    """gdn_chunk_fwd on the q/k/v blocks of y with the gates formed from a,
    b, A_log, dt_bias inside the chunk kernels.  Returns (o, ht, g, beta);
    g, beta are None unless ``want_gates``."""
    load_library()
    _req(y, "y", shape=(None, None))
    T, C = y.shape
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=y)
    N = cu_seqlens.numel() - 1
    Ta, ld = _ab_views(a, b, Hv)
    if Ta != T or a.dtype != y.dtype or a.device != y.device:
        raise ValueError("a, b must be [T, Hv] in the activation dtype, on y's device")
    _req(A_log, "A_log", torch.float32, (Hv,), device=y)
    _req(dt_bias, "dt_bias", torch.float32, (Hv,), device=y)
    _req(h0, "h0", torch.float32, (N, Hv, dk, dv), device=y)
    q, k, v = _qkv_views(y, Hk, Hv, dk, dv)
    o = out if out is not None else torch.empty((T, Hv, dv), dtype=y.dtype, device=y.device)
    _req(o, "out", y.dtype, (T, Hv, dv), device=y)
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=y.device) if want_ht else None
    g = beta = None
    if want_gates:
        g = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
        beta = torch.empty((T, Hv), dtype=torch.float32, device=y.device)
    dt = GDN_BF16 if y.dtype == torch.bfloat16 else GDN_F32
    nbytes = int(_lib.gdn_chunk_fwd_gated_workspace_size(T, N, Hk, Hv, dk, dv, dt))
    ws = _workspace(ws, nbytes, y)
    scale = dk ** -0.5 if scale is None else scale
    rc = _lib.gdn_chunk_fwd_gated(_ptr(q), _ptr(k), C, _ptr(v), C, _ptr(a), _ptr(b), ld,
                                  _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), N, T, Hk,
                                  Hv, dk, dv, float(scale), int(bool(use_qk_l2norm)), _ptr(o),
                                  _ptr(ht), _ptr(g), _ptr(beta), _ptr(ws), nbytes, _dt(y),
                                  _stream())
    _check("gdn_chunk_fwd_gated", rc)
    return o, ht, g, beta


# --------------------------------------------------------------------------
# head-sharded (Ulysses) layout: one rank's packed [q | k | v | b | a] rows
# --------------------------------------------------------------------------
def gdn_ulysses_fwd(packed, conv_w, A_log, dt_bias, cu_seqlens, Hk, Hv, dk, dv, conv_bias=None,
                    h0=None, scale=None, use_qk_l2norm=True, want_ht=False, want_gates=False,
                    ws=None):
    """packed [T, >= C + 2 Hv] rows [q | k | v | b | a] of the rank's heads
    (unit column stride, any token stride).  Returns (y [T, C], o
    [T, Hv, dv], ht or None, g or None, beta or None)."""
    load_library()
    if packed.dim() != 2 or packed.stride(1) != 1 or not packed.is_cuda:
        raise ValueError("packed must be a [T, W] GPU tensor with unit column stride")
    T, W = packed.shape
    C = 2 * Hk * dk + Hv * dv
    if W < C + 2 * Hv:
        raise ValueError("packed rows hold %d columns, [q|k|v|b|a] needs %d" % (W, C + 2 * Hv))
    _req(conv_w, "conv_w", packed.dtype, (C, None), device=packed)
    K = conv_w.shape[1]
    _req(conv_bias, "conv_bias", packed.dtype, (C,), device=packed)
    _req(A_log, "A_log", torch.float32, (Hv,), device=packed)
    _req(dt_bias, "dt_bias", torch.float32, (Hv,), device=packed)
    _req(cu_seqlens, "cu_seqlens", torch.int32, (None,), device=packed)
    N = cu_seqlens.numel() - 1
    _req(h0, "h0", torch.float32, (N, Hv, dk, dv), device=packed)
    y = torch.empty((T, C), dtype=packed.dtype, device=packed.device)
    o = torch.empty((T, Hv, dv), dtype=packed.dtype, device=packed.device)
    ht = torch.empty((N, Hv, dk, dv), dtype=torch.float32, device=packed.device) if want_ht else None
    g = beta = None
    if want_gates:
        g = torch.empty((T, Hv), dtype=torch.float32, device=packed.device)
        beta = torch.empty((T, Hv), dtype=torch.float32, device=packed.device)
    dt = _dt(packed)
    nbytes = int(_lib.gdn_ulysses_fwd_workspace_size(T, N, Hk, Hv, dk, dv, dt))
    ws = _workspace(ws, nbytes, packed)
    scale = dk ** -0.5 if scale is None else scale
    rc = _lib.gdn_ulysses_fwd(_ptr(packed), packed.stride(0), _ptr(conv_w), _ptr(conv_bias), K,
                              _ptr(A_log), _ptr(dt_bias), _ptr(h0), _ptr(cu_seqlens), N, T, Hk, Hv,
                              dk, dv, float(scale), int(bool(use_qk_l2norm)), _ptr(y), _ptr(o),
                              _ptr(ht), _ptr(g), _ptr(beta), _ptr(ws), nbytes, dt, _stream())
    _check("gdn_ulysses_fwd", rc)
    return y, o, ht, g, beta
