// chunk_summary.hip -- a shard's affine state summary and the prefix merge of
// summaries: the per-rank compute that the page's context-parallel state
// exchange passes around (hyper-parallel "linear_attention_context_parallel.py",
// _compute_gdn_state_summary_from_prepared, _merge_gdn_prefix_state_summaries_torch,
// _apply_gdn_state_summary).  The kernels are in chunk_loop.h.
#include <hip/hip_runtime.h>

#include "chunk_loop.h"
#include "gdn_internal.h"

using namespace gdn_chunk;

namespace {

Plan summary_plan(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  return make_plan(T, N, Hv, dk, dv, gdn::chunk_rec_bytes(dt), true);
}

template <typename E>
int dispatch(int dk, int dv, const LoopArgs& a, const int32_t* cu, int N, int64_t T, const Plan& pl,
             char* ws, float* M, float* Ev, hipStream_t stream) {
#define GDN_CASE(K_, V_) \
  if (dk == K_ && dv == V_) return run_summary<E, K_, V_>(a, cu, N, T, pl, ws, M, Ev, stream);
  if constexpr (sizeof(E) == 2) {
    GDN_CASE(128, 128)
    GDN_CASE(128, 64)
    GDN_CASE(64, 128)
    GDN_CASE(128, 32)
    GDN_CASE(32, 128)
  }
  GDN_CASE(64, 64)
  GDN_CASE(32, 32)
  GDN_CASE(64, 32)
  GDN_CASE(32, 64)
#undef GDN_CASE
  return gdn::fail(GDN_EUNSUPPORTED, "gdn_chunk_summary: dk=%d dv=%d has no kernel for this dtype", dk, dv);
}

template <int DK>
int merge_dispatch(int dv, const float* M, const float* E, int R, int S, const float* h_in,
                   float* h_out, hipStream_t stream) {
#define GDN_MCASE(V_)                                                                             \
  if (dv == V_) {                                                                                 \
    hipLaunchKernelGGL((merge_summaries_kernel<DK, V_>), dim3(S, V_ / 16), dim3(DK * 2), 0, stream, \
                       M, E, R, S, h_in, h_out);                                                  \
    return gdn::check_launch("gdn_merge_summaries");                                              \
  }
  GDN_MCASE(32)
  GDN_MCASE(64)
  GDN_MCASE(128)
#undef GDN_MCASE
  return gdn::fail(GDN_EUNSUPPORTED, "gdn_merge_summaries: dv=%d", dv);
}

}  // namespace

extern "C" size_t gdn_chunk_summary_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                                   int32_t dk, int32_t dv, gdn_dtype dt) {
  (void)Hk;
  if (T < 0 || N < 0 || Hv < 1 || dk < 1 || dv < 1) return 0;
  return summary_plan(T, N, Hv, dk, dv, dt).end;
}

extern "C" int gdn_chunk_summary(const void* k, int64_t ld_k, const void* v, int64_t ld_v,
                                 const float* g, const float* beta, const int32_t* cu_seqlens,
                                 int32_t N, int64_t T, int32_t Hk, int32_t Hv, int32_t dk,
                                 int32_t dv, int use_qk_l2norm, float* M, float* E, void* ws,
                                 size_t ws_bytes, gdn_dtype dt, hipStream_t stream) {
  int rc = gdn::validate_chunk("gdn_chunk_summary", k, k, ld_k, v, ld_v, g, beta, cu_seqlens, N, T,
                               Hk, Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  if (N > 0 && !cu_seqlens) return gdn::fail(GDN_EINVAL, "gdn_chunk_summary: null cu_seqlens");
  if ((M && !gdn::aligned16(M)) || (E && !gdn::aligned16(E)))
    return gdn::fail(GDN_EINVAL, "gdn_chunk_summary: M and E must be 16-byte aligned");
  if (N == 0 || (!M && !E)) return GDN_OK;
  const Plan pl = summary_plan(T, N, Hv, dk, dv, dt);
  if (!ws || ws_bytes < pl.end || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "gdn_chunk_summary: workspace needs %zu bytes, 256-byte aligned",
                     pl.end);
  LoopArgs a{};
  a.q = k;
  a.k = k;
  a.ld_qk = ld_k;
  a.v = v;
  a.ld_v = ld_v;
  a.g = g;
  a.beta = beta;
  a.Hk = Hk;
  a.Hv = Hv;
  a.scale = 1.f;
  a.use_l2norm = use_qk_l2norm ? 1 : 0;
  return dt == GDN_BF16 ? dispatch<bf16>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, M, E, stream)
                        : dispatch<float>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, M, E, stream);
}

extern "C" int gdn_merge_summaries(const float* M, const float* E, int32_t R, int32_t S, int32_t dk,
                                   int32_t dv, const float* h_in, float* h_out, hipStream_t stream) {
  if (R < 0 || S < 0) return gdn::fail(GDN_EINVAL, "gdn_merge_summaries: negative R or S");
  const bool dims = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
  if (!dims) return gdn::fail(GDN_EUNSUPPORTED, "gdn_merge_summaries: dk=%d dv=%d", dk, dv);
  if (S == 0) return GDN_OK;
  if (!h_out || (R > 0 && (!M || !E)))
    return gdn::fail(GDN_EINVAL, "gdn_merge_summaries: null pointer");
  if (!gdn::aligned16(M) || !gdn::aligned16(E) || !gdn::aligned16(h_in) || !gdn::aligned16(h_out))
    return gdn::fail(GDN_EINVAL, "gdn_merge_summaries: pointers must be 16-byte aligned");
  if (dk == 128) return merge_dispatch<128>(dv, M, E, R, S, h_in, h_out, stream);
  if (dk == 64) return merge_dispatch<64>(dv, M, E, R, S, h_in, h_out, stream);
  return merge_dispatch<32>(dv, M, E, R, S, h_in, h_out, stream);
}
