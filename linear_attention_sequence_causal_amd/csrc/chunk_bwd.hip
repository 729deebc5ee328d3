// chunk_bwd.hip -- chunked gated delta rule, backward (reverse mode of
// gdn_chunk_fwd).
#include <hip/hip_runtime.h>

#include "chunk_common.h"
#include "gdn_internal.h"

size_t gdn_chunk_fwd_workspace(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv);

namespace gdn {
int validate_chunk(const char* fn, const void* q, const void* k, int64_t ld_qk, const void* v,
                   int64_t ld_v, const float* g, const float* beta, const int32_t* cu, int32_t N,
                   int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt);
}

extern "C" size_t gdn_chunk_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                           int32_t dk, int32_t dv, gdn_dtype dt, int bwd) {
  (void)Hk;
  (void)dt;
  if (bwd) return 0;
  return gdn_chunk_fwd_workspace(T, N, Hv, dk, dv);
}

extern "C" int gdn_chunk_bwd(const void* q, const void* k, int64_t ld_qk, const void* v,
                             int64_t ld_v, const float* g, const float* beta, const float* h0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                             int32_t Hv, int32_t dk, int32_t dv, float scale, int use_qk_l2norm,
                             const void* d_o, const float* dht, void* dq, void* dk_,
                             int64_t ld_dqk, void* dv_, int64_t ld_dv, float* dg, float* dbeta,
                             float* dh0, void* ws, size_t ws_bytes, gdn_dtype dt,
                             hipStream_t stream) {
  (void)h0; (void)scale; (void)use_qk_l2norm; (void)d_o; (void)dht; (void)dq; (void)dk_;
  (void)ld_dqk; (void)dv_; (void)ld_dv; (void)dg; (void)dbeta; (void)dh0; (void)ws;
  (void)ws_bytes; (void)stream;
  int rc = gdn::validate_chunk("gdn_chunk_bwd", q, k, ld_qk, v, ld_v, g, beta, cu_seqlens, N, T, Hk,
                               Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  return gdn::fail(GDN_EUNSUPPORTED, "gdn_chunk_bwd: not built yet");
}
