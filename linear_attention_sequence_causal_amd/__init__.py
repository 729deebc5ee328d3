"""MI355X (gfx950) hot path of a context-parallel Gated DeltaNet token mixer.

The compute lives in ``libgdn.so`` (hand-written HIP, C ABI in
``include/gdn.h``); ``gdn`` is its thin torch binding and ``workloads`` the
seeded synthetic inputs of the benchmark workloads.
"""
from . import gdn  # noqa: F401
from .gdn import (  # noqa: F401
    gdn_chunk_bwd,
    gdn_chunk_fwd,
    gdn_conv1d_silu_halo,
    gdn_conv1d_silu_halo_bwd,
    gdn_localize_cu_seqlens,
    load_library,
    make_meta,
    read_meta,
)
