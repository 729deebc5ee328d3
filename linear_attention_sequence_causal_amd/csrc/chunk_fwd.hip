// chunk_fwd.hip -- gdn_chunk_fwd: the chunked gated delta rule forward
// (hyper-parallel "linear_attention_context_parallel.py", _l2norm_torch,
// _prepare_gdn_chunks_for_summary, _run_prepared_gdn_chunks), per sequence of
// cu_seqlens; the kernels are in chunk_loop.h.
#include <hip/hip_runtime.h>

#include "chunk_loop.h"
#include "gdn_internal.h"

using namespace gdn_chunk;

namespace {

template <typename E, int DK, int DV>
int launch_fwd(const LoopArgs& a, const int32_t* cu, int N, int64_t T, const Plan& pl, char* ws,
               hipStream_t stream) {
  if (N > 0 && a.ht) {
    hipLaunchKernelGGL(empty_seq_state_kernel, dim3(N, a.Hv), dim3(256), 0, stream, cu, a.h0, a.ht,
                       a.Hv, DK * DV);
    if (int rc = gdn::check_launch("gdn_chunk_fwd(empty)")) return rc;
  }
  if (T == 0 || N == 0) return GDN_OK;
  return run_pipeline<E, DK, DV, kOut>(a, cu, N, T, pl, ws, false, stream);
}

template <typename E>
int dispatch(int dk, int dv, const LoopArgs& a, const int32_t* cu, int N, int64_t T, const Plan& pl,
             char* ws, hipStream_t stream) {
#define GDN_CASE(K_, V_) \
  if (dk == K_ && dv == V_) return launch_fwd<E, K_, V_>(a, cu, N, T, pl, ws, stream);
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
  return gdn::fail(GDN_EUNSUPPORTED, "gdn_chunk_fwd: dk=%d dv=%d has no kernel for this dtype", dk, dv);
}

}  // namespace

namespace gdn {
// argument validation shared by the chunk entry points
int validate_chunk(const char* fn, const void* q, const void* k, int64_t ld_qk, const void* v,
                   int64_t ld_v, const float* g, const float* beta, const int32_t* cu, int32_t N,
                   int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  if (T < 0 || N < 0) return fail(GDN_EINVAL, "%s: negative T or N", fn);
  if (T > INT32_MAX) return fail(GDN_EINVAL, "%s: T must be < 2^31", fn);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_EINVAL, "%s: need Hk >= 1 and Hv %% Hk == 0 (Hk=%d Hv=%d)", fn, Hk, Hv);
  if (dt != GDN_F32 && dt != GDN_BF16) return fail(GDN_EINVAL, "%s: unknown dtype", fn);
  const bool dims = (dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128);
  if (!dims || (dt == GDN_F32 && (dk > 64 || dv > 64)))
    return fail(GDN_EUNSUPPORTED, "%s: dk=%d dv=%d has no kernel for this dtype", fn, dk, dv);
  if (ld_qk < (int64_t)Hk * dk || ld_v < (int64_t)Hv * dv)
    return fail(GDN_EINVAL, "%s: row strides smaller than the head blocks", fn);
  const int es = dt == GDN_BF16 ? 2 : 4;
  if ((ld_qk * es) % 16 || (ld_v * es) % 16)
    return fail(GDN_EINVAL, "%s: row strides must be multiples of 16 bytes", fn);
  // a chunk's 64 rows (q, k, v and o) are addressed with 32-bit byte offsets
  const int64_t lim = (int64_t)1 << 32;
  if (64 * ld_qk * es >= lim || 64 * ld_v * es >= lim || 64 * (int64_t)Hv * dv * es >= lim)
    return fail(GDN_EINVAL, "%s: 64 rows of q, k, v or o must span less than 4 GiB", fn);
  if (T > 0) {
    if (N < 1) return fail(GDN_EINVAL, "%s: T > 0 needs N >= 1 sequences", fn);
    if (!q || !k || !v || !g || !beta || !cu) return fail(GDN_EINVAL, "%s: null pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
      return fail(GDN_EINVAL, "%s: q, k, v must be 16-byte aligned", fn);
  }
  return GDN_OK;
}

// bytes of the prepared record per (chunk, value head): bfloat16 only
size_t chunk_rec_bytes(gdn_dtype dt) { return dt == GDN_BF16 ? (size_t)kRecBytes : 0; }

// the summary pass can run first segments in the output mode (same block shape)
bool chunk_first_out(int32_t dk, int32_t dv, gdn_dtype dt) { return dt == GDN_BF16 && dk == 128 && dv == 128; }

size_t chunk_fwd_workspace(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  if (T < 0 || N < 0 || Hv < 1) return 0;
  return make_plan(T, N, Hv, dk, dv, chunk_rec_bytes(dt), chunk_first_out(dk, dv, dt)).end;
}
}  // namespace gdn

extern "C" int gdn_chunk_fwd(const void* q, const void* k, int64_t ld_qk, const void* v,
                             int64_t ld_v, const float* g, const float* beta, const float* h0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                             int32_t Hv, int32_t dk, int32_t dv, float scale, int use_qk_l2norm,
                             void* o, float* ht, void* ws, size_t ws_bytes, gdn_dtype dt,
                             hipStream_t stream) {
  int rc = gdn::validate_chunk("gdn_chunk_fwd", q, k, ld_qk, v, ld_v, g, beta, cu_seqlens, N, T, Hk,
                               Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  if (T > 0 && !o) return gdn::fail(GDN_EINVAL, "gdn_chunk_fwd: o is null");
  if (T > 0 && !gdn::aligned16(o)) return gdn::fail(GDN_EINVAL, "gdn_chunk_fwd: o must be 16-byte aligned");
  if (N > 0 && ht && !cu_seqlens) return gdn::fail(GDN_EINVAL, "gdn_chunk_fwd: null cu_seqlens");
  const Plan pl = make_plan(T, N, Hv, dk, dv, gdn::chunk_rec_bytes(dt), gdn::chunk_first_out(dk, dv, dt));
  if (!ws || ws_bytes < pl.end || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "gdn_chunk_fwd: workspace needs %zu bytes, 256-byte aligned",
                     pl.end);
  LoopArgs a{};
  a.q = q;
  a.k = k;
  a.ld_qk = ld_qk;
  a.v = v;
  a.ld_v = ld_v;
  a.g = g;
  a.beta = beta;
  a.h0 = h0;
  a.Hk = Hk;
  a.Hv = Hv;
  a.scale = scale;
  a.use_l2norm = use_qk_l2norm ? 1 : 0;
  a.o = o;
  a.ht = ht;
  return dt == GDN_BF16 ? dispatch<bf16>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream)
                        : dispatch<float>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream);
}
