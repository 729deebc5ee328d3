// ulysses.hip -- gdn_ulysses_fwd: one rank's compute in the head-sharded
// (Ulysses) layout of the hyper-parallel page (LinearAttentionUlyssesCPWrapper:
// after _seq_to_head_qkvba every rank holds the whole sequence for its slice
// of the heads, as packed rows [q | k | v | b | a]; it runs the conv over its
// local channel slices, forms the gates from its b and a columns with its
// slices of A_log and dt_bias, and runs the gated delta rule on its heads).
// The steps are the library's own kernels: the conv reads the q|k|v columns
// of the packed rows in place, the chunk forward forms the gates from the b|a
// columns inside its prep.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

extern "C" size_t gdn_ulysses_fwd_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                                 int32_t dk, int32_t dv, gdn_dtype dt) {
  return gdn_chunk_fwd_gated_workspace_size(T, N, Hk, Hv, dk, dv, dt);
}

extern "C" int gdn_ulysses_fwd(const void* packed, int64_t ld_packed, const void* conv_w,
                               const void* conv_bias, int32_t K, const float* A_log,
                               const float* dt_bias, const float* h0, const int32_t* cu_seqlens,
                               int32_t N, int64_t T, int32_t Hk, int32_t Hv, int32_t dk,
                               int32_t dv, float scale, int use_qk_l2norm, void* y, void* o,
                               float* ht, float* g_out, float* beta_out, void* ws,
                               size_t ws_bytes, gdn_dtype dt, hipStream_t stream) {
  const char* fn = "gdn_ulysses_fwd";
  if (Hk < 1 || Hv < 1 || dk < 1 || dv < 1 || T < 0)
    return gdn::fail(GDN_EINVAL, "%s: bad head counts, head sizes or T", fn);
  if (dt != GDN_F32 && dt != GDN_BF16) return gdn::fail(GDN_EINVAL, "%s: unknown dtype", fn);
  const int64_t C = 2 * (int64_t)Hk * dk + (int64_t)Hv * dv;
  if (C > INT32_MAX) return gdn::fail(GDN_EINVAL, "%s: too many channels", fn);
  if (ld_packed < C + 2 * (int64_t)Hv)
    return gdn::fail(GDN_EINVAL, "%s: packed rows shorter than [q|k|v|b|a] (%lld < %lld)", fn,
                     (long long)ld_packed, (long long)(C + 2 * (int64_t)Hv));
  if (T > 0 && (!packed || !y)) return gdn::fail(GDN_EINVAL, "%s: null packed rows or y", fn);
  // the chunk forward's checks (workspace included) run before anything is launched
  const size_t need = gdn_ulysses_fwd_workspace_size(T, N, Hk, Hv, dk, dv, dt);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn, need);
  const size_t es = dt == GDN_BF16 ? 2 : 4;
  const char* base = static_cast<const char*>(packed);
  const void* b_cols = base + (size_t)C * es;
  const void* a_cols = base + (size_t)(C + Hv) * es;
  char* yc = static_cast<char*>(y);
  const void* q = yc;
  const void* k = yc + (size_t)Hk * dk * es;
  const void* v = yc + (size_t)2 * Hk * dk * es;
  // validate the chunk call on its real arguments first (no launch happens
  // if it would fail), then run the conv and the chunk
  int rc = gdn::validate_chunk(fn, q, k, C, v, C, (const float*)a_cols, (const float*)b_cols,
                               cu_seqlens, N, T, Hk, Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  if (T > 0 && (!A_log || !dt_bias || !o)) return gdn::fail(GDN_EINVAL, "%s: null pointer", fn);
  if ((rc = gdn::conv_fwd_strided(packed, ld_packed, conv_w, conv_bias, nullptr, cu_seqlens, N, T,
                                  (int32_t)C, K, nullptr, y, dt, stream)) != GDN_OK)
    return rc;
  return gdn_chunk_fwd_gated(q, k, C, v, C, a_cols, b_cols, ld_packed, A_log, dt_bias, h0,
                             cu_seqlens, N, T, Hk, Hv, dk, dv, scale, use_qk_l2norm, o, ht, g_out,
                             beta_out, ws, ws_bytes, dt, stream);
}
