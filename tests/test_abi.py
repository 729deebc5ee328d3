"""The C-ABI library loads on a machine without a GPU, exports every entry
point declared in include/gdn.h, and rejects invalid host-visible arguments
with the documented status codes before touching the device."""
import ctypes
import os
import re

import pytest

from linear_attention_sequence_causal_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(gdn_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built; run `python -m linear_attention_sequence_causal_amd.build`")
    return gdn.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gdn_localize_cu_seqlens", "gdn_conv1d_silu_halo", "gdn_conv1d_silu_halo_bwd",
              "gdn_chunk_fwd", "gdn_chunk_bwd", "gdn_chunk_workspace_size",
              "gdn_conv_bwd_workspace_size", "gdn_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(gdn.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    assert set(declared_functions()) == set(gdn.ENTRY_POINTS)


def test_meta_struct_size():
    # 3 int64 + 8 int32, no padding
    assert gdn.META_BYTES == 56


P = None


def test_localize_rejects_bad_arguments(lib):
    fake = ctypes.c_void_p(0x1000)
    bad = [
        (fake, 0, 16, 1, 0, 4),     # num_seqs < 1
        (fake, 2, 16, 0, 0, 4),     # world_size < 1
        (fake, 2, 16, 2, 2, 4),     # rank out of range
        (fake, 2, 16, 2, -1, 4),
        (fake, 2, 16, 2, 0, 0),     # K < 1
        (fake, 2, 0, 1, 0, 4),      # no tokens
        (fake, 2, 17, 2, 0, 4),     # remainder
    ]
    for args in bad:
        rc = lib.gdn_localize_cu_seqlens(*args, fake, fake, None)
        assert rc == gdn.GDN_EINVAL, args
        assert lib.gdn_last_error().decode()
    assert lib.gdn_localize_cu_seqlens(None, 2, 16, 2, 0, 4, fake, fake, None) == gdn.GDN_EINVAL


def test_conv_rejects_bad_arguments(lib):
    f = ctypes.c_void_p(0x1000)
    # K out of range, C < 1, negative T, null x with T > 0, unknown dtype
    assert lib.gdn_conv1d_silu_halo(f, f, None, None, f, 1, 10, 8, 9, None, f, 1, None) == gdn.GDN_EINVAL
    assert lib.gdn_conv1d_silu_halo(f, f, None, None, f, 1, 10, 0, 4, None, f, 1, None) == gdn.GDN_EINVAL
    assert lib.gdn_conv1d_silu_halo(f, f, None, None, f, 1, -1, 8, 4, None, f, 1, None) == gdn.GDN_EINVAL
    assert lib.gdn_conv1d_silu_halo(None, f, None, None, f, 1, 10, 8, 4, None, f, 1, None) == gdn.GDN_EINVAL
    assert lib.gdn_conv1d_silu_halo(f, f, None, None, f, 1, 10, 8, 4, None, f, 7, None) == gdn.GDN_EINVAL
    # T = 0 is a no-op
    assert lib.gdn_conv1d_silu_halo(None, None, None, None, None, 0, 0, 8, 4, None, None, 1, None) == gdn.GDN_OK
    # backward: workspace too small
    need = lib.gdn_conv_bwd_workspace_size(100, 64, 4)
    assert need > 0
    rc = lib.gdn_conv1d_silu_halo_bwd(f, f, None, None, f, 1, 100, 64, 4, None, f, f, f, None, None,
                                      f, need - 1, 1, None)
    assert rc == gdn.GDN_EWORKSPACE


def _chunk(lib, **kw):
    f = ctypes.c_void_p(0x1000)
    a = dict(q=f, k=f, ld_qk=6144, v=f, ld_v=6144, g=f, beta=f, h0=None, cu=f, N=1, T=64, Hk=16,
             Hv=16, dk=128, dv=128, scale=0.1, l2=1, o=f, ht=None, ws=f, ws_bytes=1 << 40, dt=1)
    a.update(kw)
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["ld_qk"], a["v"], a["ld_v"], a["g"], a["beta"],
                             a["h0"], a["cu"], a["N"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                             a["scale"], a["l2"], a["o"], a["ht"], a["ws"], a["ws_bytes"], a["dt"],
                             None)


def test_chunk_rejects_bad_arguments(lib):
    assert _chunk(lib, Hv=24, Hk=16) == gdn.GDN_EINVAL          # Hv % Hk
    assert _chunk(lib, Hk=0) == gdn.GDN_EINVAL
    assert _chunk(lib, dk=48) == gdn.GDN_EUNSUPPORTED
    assert _chunk(lib, dv=256) == gdn.GDN_EUNSUPPORTED
    assert _chunk(lib, dt=0) == gdn.GDN_EUNSUPPORTED             # fp32 at d = 128
    assert _chunk(lib, ld_qk=100) == gdn.GDN_EINVAL              # stride below the head block
    assert _chunk(lib, ld_qk=2049 + 2048, ld_v=6144) == gdn.GDN_EINVAL  # not 16-byte multiple
    assert _chunk(lib, q=None) == gdn.GDN_EINVAL
    assert _chunk(lib, q=ctypes.c_void_p(0x1002)) == gdn.GDN_EINVAL     # misaligned
    assert _chunk(lib, T=-1) == gdn.GDN_EINVAL
    assert _chunk(lib, ld_qk=1 << 25, ld_v=6144) == gdn.GDN_EINVAL  # 64 rows past 32-bit offsets
    assert _chunk(lib, ws=None, ws_bytes=0) == gdn.GDN_EWORKSPACE
    assert _chunk(lib, ws=ctypes.c_void_p(0x1010)) == gdn.GDN_EWORKSPACE  # not 256-aligned
    assert _chunk(lib, ws_bytes=16) == gdn.GDN_EWORKSPACE
    assert b"workspace" in lib.gdn_last_error()


def test_saved_pair_rejects_bad_buffers(lib):
    """gdn_chunk_fwd_save / gdn_chunk_bwd_saved: the saved buffer is checked
    (null, short, misaligned) before anything is launched."""
    f = ctypes.c_void_p(0x1000)
    need = lib.gdn_chunk_saved_size(64, 1, 16, 16, 128, 128, 1)
    # records (7424 B per chunk and head) and bf16 states, 3 chunk slots
    assert need >= 3 * 16 * (7424 + 2 * 128 * 128)
    assert lib.gdn_chunk_saved_size(64, 1, 16, 16, 64, 64, 0) >= 3 * 16 * 4 * 64 * 64
    assert lib.gdn_chunk_saved_size(-1, 1, 16, 16, 128, 128, 1) == 0

    def fwd(saved, nbytes):
        return lib.gdn_chunk_fwd_save(f, f, 6144, f, 6144, f, f, None, f, 1, 64, 16, 16, 128, 128,
                                      0.1, 1, f, None, saved, nbytes, f, 1 << 40, 1, None)

    def bwd(saved, nbytes):
        return lib.gdn_chunk_bwd_saved(f, f, 6144, f, 6144, f, f, None, f, 1, 64, 16, 16, 128, 128,
                                       0.1, 1, f, None, f, f, 6144, f, 2048, f, f, None, saved,
                                       nbytes, f, 1 << 40, 1, None)
    assert fwd(None, 0) == gdn.GDN_EWORKSPACE
    assert fwd(f, need - 1) == gdn.GDN_EWORKSPACE
    assert fwd(ctypes.c_void_p(0x1010), need) == gdn.GDN_EWORKSPACE
    assert b"saved" in lib.gdn_last_error()
    assert bwd(None, 0) == gdn.GDN_EINVAL
    assert bwd(f, need - 1) == gdn.GDN_EINVAL
    assert bwd(ctypes.c_void_p(0x1010), need) == gdn.GDN_EINVAL
    assert b"saved" in lib.gdn_last_error()


def test_workspace_sizes_are_host_only(lib):
    # sizes are pure host arithmetic; segment summaries appear for long sequences
    small = lib.gdn_chunk_workspace_size(256, 1, 2, 2, 32, 32, 0, 0)
    big = lib.gdn_chunk_workspace_size(131072, 1, 16, 32, 128, 128, 1, 0)
    assert 0 < small < big
    assert lib.gdn_conv_bwd_workspace_size(0, 64, 4) == 0


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 300, 4097, 131072])
@pytest.mark.parametrize("N", [1, 2])
def test_workspace_size_edge_lengths(lib, T, N):
    """The host plan (segment lengths, capacities) is total arithmetic for
    empty, sub-chunk and long inputs, forward and backward, both dtypes."""
    for dt, d in ((0, 32), (1, 128)):
        for bwd in (0, 1):
            size = lib.gdn_chunk_workspace_size(T, N, 2, 4, d, d, dt, bwd)
            assert size >= 0
            if T > 0:
                assert size > 0


def _chunk_bwd(lib, **kw):
    f = ctypes.c_void_p(0x1000)
    a = dict(q=f, k=f, ld_qk=6144, v=f, ld_v=6144, g=f, beta=f, h0=None, cu=f, N=1, T=64, Hk=16,
             Hv=16, dk=128, dv=128, scale=0.1, l2=1, do=f, dht=None, dq=f, dk_=f, ld_dqk=6144,
             dv_=f, ld_dv=6144, dg=f, dbeta=f, dh0=None, ws=f, ws_bytes=1 << 40, dt=1)
    a.update(kw)
    return lib.gdn_chunk_bwd(a["q"], a["k"], a["ld_qk"], a["v"], a["ld_v"], a["g"], a["beta"],
                             a["h0"], a["cu"], a["N"], a["T"], a["Hk"], a["Hv"], a["dk"], a["dv"],
                             a["scale"], a["l2"], a["do"], a["dht"], a["dq"], a["dk_"], a["ld_dqk"],
                             a["dv_"], a["ld_dv"], a["dg"], a["dbeta"], a["dh0"], a["ws"],
                             a["ws_bytes"], a["dt"], None)


def test_chunk_bwd_rejects_shapes_it_has_no_kernel_for(lib):
    """The backward's kernels cover dk == dv with d in {64, 128} (bfloat16)
    or {32, 64} (float32); shapes the forward accepts beyond that are
    reported as unsupported, not run."""
    assert _chunk_bwd(lib, dk=128, dv=64, ld_qk=4096, ld_v=4096) == gdn.GDN_EUNSUPPORTED
    assert _chunk_bwd(lib, dk=64, dv=128, ld_qk=2048, ld_v=4096) == gdn.GDN_EUNSUPPORTED
    assert _chunk_bwd(lib, dk=32, dv=32, ld_qk=1024, ld_v=1024) == gdn.GDN_EUNSUPPORTED  # bf16 d=32
    assert b"dk == dv" in lib.gdn_last_error()
    assert _chunk_bwd(lib, dk=128, dv=128, dt=0) == gdn.GDN_EUNSUPPORTED  # fp32 d=128
    assert _chunk_bwd(lib, dq=None) == gdn.GDN_EINVAL
    assert _chunk_bwd(lib, dg=None) == gdn.GDN_EINVAL
    assert _chunk_bwd(lib, ld_dqk=100) == gdn.GDN_EINVAL
    assert _chunk_bwd(lib, ld_dqk=1 << 25) == gdn.GDN_EINVAL   # 64 rows past 32-bit offsets
    assert b"4 GiB" in lib.gdn_last_error()
    assert _chunk_bwd(lib, ld_dv=1 << 25) == gdn.GDN_EINVAL
    assert _chunk_bwd(lib, ws_bytes=16) == gdn.GDN_EWORKSPACE


def test_segment_hook_is_thread_local_and_not_public(lib):
    """Forcing the segment length is a test hook that the public header does
    not declare; it changes only the calling thread's plans and is undone by
    setting 0."""
    import threading
    assert "gdn_testing_set_segment_chunks" not in declared_functions()
    fn = lib.gdn_testing_set_segment_chunks
    fn.argtypes = [ctypes.c_int]
    fn.restype = ctypes.c_int
    base = lib.gdn_chunk_workspace_size(4096, 1, 2, 4, 128, 128, 1, 0)
    assert fn(1) == 0
    forced = lib.gdn_chunk_workspace_size(4096, 1, 2, 4, 128, 128, 1, 0)
    other = []
    t = threading.Thread(target=lambda: other.append(
        lib.gdn_chunk_workspace_size(4096, 1, 2, 4, 128, 128, 1, 0)))
    t.start()
    t.join()
    assert fn(0) == 1
    assert forced != base and other == [base]
    assert lib.gdn_chunk_workspace_size(4096, 1, 2, 4, 128, 128, 1, 0) == base
