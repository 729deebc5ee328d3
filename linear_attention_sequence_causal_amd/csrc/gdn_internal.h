// gdn_internal.h -- host-side helpers shared by the libgdn sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "gdn.h"

namespace gdn {

// Records a formatted message as the thread's last error and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GDN_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Segment length (in 64-token chunks) forced on the chunk plans of the
// calling thread, 0 for the plan's own choice.  Set only through
// gdn_testing_set_segment_chunks, which the public header does not declare:
// it exists so that tests can run the segment machinery on small inputs.
int segment_chunks_override();

// Shared by the chunk entry points (defined in chunk_fwd.hip): argument
// checks of a chunk call, the forward's workspace size and the bytes of the
// prepared record per (chunk, value head).
int validate_chunk(const char* fn, const void* q, const void* k, int64_t ld_qk, const void* v,
                   int64_t ld_v, const float* g, const float* beta, const int32_t* cu, int32_t N,
                   int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt);
size_t chunk_fwd_workspace(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt);
size_t chunk_rec_bytes(gdn_dtype dt);

// The buffer a saving forward (gdn_chunk_fwd_save) fills for the backward
// (gdn_chunk_bwd_saved): the prepared records ([chunk_cap][Hv] x
// chunk_rec_bytes, bfloat16 only) and the state entering every chunk
// ([chunk_cap][Hv][dk][dv] activations), each 256-byte aligned.
struct SavedLayout {
  size_t off_rec, off_states, end;
};
SavedLayout chunk_saved_layout(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv,
                               gdn_dtype dt);

// The forward conv with an x token stride (conv.hip).
int conv_fwd_strided(const void* x, int64_t ldx, const void* w, const void* bias,
                     const void* halo, const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t C,
                     int32_t K, const gdn_cp_meta* meta, void* y, gdn_dtype dt, hipStream_t stream);

}  // namespace gdn
