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
               hipStream_t stream, char* rec_buf) {
  // a saving forward (states set) stores the state entering every chunk
  if (N > 0 && a.ht) {
    hipLaunchKernelGGL(empty_seq_state_kernel, dim3(N, a.Hv), dim3(256), 0, stream, cu, a.h0, a.ht,
                       a.Hv, DK * DV);
    if (int rc = gdn::check_launch("gdn_chunk_fwd(empty)")) return rc;
  }
  if (T == 0 || N == 0) return GDN_OK;
  if (a.states) return run_pipeline<E, DK, DV, kOutSave>(a, cu, N, T, pl, ws, false, stream, rec_buf);
  return run_pipeline<E, DK, DV, kOut>(a, cu, N, T, pl, ws, false, stream, rec_buf);
}

template <typename E>
int dispatch(int dk, int dv, const LoopArgs& a, const int32_t* cu, int N, int64_t T, const Plan& pl,
             char* ws, hipStream_t stream, char* rec_buf = nullptr) {
#define GDN_CASE(K_, V_) \
  if (dk == K_ && dv == V_) return launch_fwd<E, K_, V_>(a, cu, N, T, pl, ws, stream, rec_buf);
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

size_t chunk_fwd_workspace(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  if (T < 0 || N < 0 || Hv < 1) return 0;
  return make_plan(T, N, Hv, dk, dv, chunk_rec_bytes(dt)).end;
}

SavedLayout chunk_saved_layout(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv,
                               gdn_dtype dt) {
  // every plan of these sizes has the same chunk capacity and chunk order
  const size_t cap = (size_t)make_plan(T, N, Hv, dk, dv, 0).chunk_cap;
  const size_t es = dt == GDN_BF16 ? 2 : 4;
  SavedLayout L;
  L.off_rec = 0;
  L.off_states = round_up(chunk_rec_bytes(dt) * cap * Hv, 256);
  L.end = round_up(L.off_states + es * cap * Hv * dk * dv, 256);
  return L;
}

// gdn_gating_fwd's kernel on a stream (gating.hip)
int launch_gating_fwd(const void* a, const void* b, int64_t ld, const float* A_log,
                      const float* dt_bias, int64_t T, int32_t Hv, float* g, float* beta,
                      gdn_dtype dt, hipStream_t stream);
}  // namespace gdn

namespace {

// whether (dt, dk, dv) runs the prepared-chunk path (whose prep reads the gates)
bool prep_path(gdn_dtype dt, int dk, int dv) {
  if (dt != GDN_BF16) return false;
#define GDN_PCASE(K_, V_) \
  if (dk == K_ && dv == V_) return uses_prep<bf16, K_, V_, kOut>();
  GDN_PCASE(128, 128)
  GDN_PCASE(128, 64)
  GDN_PCASE(64, 128)
  GDN_PCASE(128, 32)
  GDN_PCASE(32, 128)
  GDN_PCASE(64, 64)
  GDN_PCASE(32, 32)
  GDN_PCASE(64, 32)
  GDN_PCASE(32, 64)
#undef GDN_PCASE
  return false;
}

LoopArgs loop_args(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                   const float* g, const float* beta, const float* h0, int32_t Hk, int32_t Hv,
                   float scale, int use_qk_l2norm, void* o, float* ht) {
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
  return a;
}

int check_out(const char* fn, void* o, float* ht, int32_t N, int64_t T, const int32_t* cu) {
  if (T > 0 && !o) return gdn::fail(GDN_EINVAL, "%s: o is null", fn);
  if (T > 0 && !gdn::aligned16(o)) return gdn::fail(GDN_EINVAL, "%s: o must be 16-byte aligned", fn);
  if (N > 0 && ht && !cu) return gdn::fail(GDN_EINVAL, "%s: null cu_seqlens", fn);
  return GDN_OK;
}

Plan fwd_plan(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  return make_plan(T, N, Hv, dk, dv, gdn::chunk_rec_bytes(dt));
}

// the gated forward's gate buffers (g, beta [T, Hv] float32) after the plan,
// when its kernels read given gates
size_t gated_extra(int64_t T, int32_t Hv, gdn_dtype dt, int32_t dk, int32_t dv) {
  return prep_path(dt, dk, dv) ? 0 : 2 * gdn::round_up(sizeof(float) * (size_t)T * Hv, 256);
}

}  // namespace

extern "C" int gdn_chunk_fwd(const void* q, const void* k, int64_t ld_qk, const void* v,
                             int64_t ld_v, const float* g, const float* beta, const float* h0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                             int32_t Hv, int32_t dk, int32_t dv, float scale, int use_qk_l2norm,
                             void* o, float* ht, void* ws, size_t ws_bytes, gdn_dtype dt,
                             hipStream_t stream) {
  int rc = gdn::validate_chunk("gdn_chunk_fwd", q, k, ld_qk, v, ld_v, g, beta, cu_seqlens, N, T, Hk,
                               Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  if ((rc = check_out("gdn_chunk_fwd", o, ht, N, T, cu_seqlens)) != GDN_OK) return rc;
  const Plan pl = fwd_plan(T, N, Hv, dk, dv, dt);
  if (!ws || ws_bytes < pl.end || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "gdn_chunk_fwd: workspace needs %zu bytes, 256-byte aligned",
                     pl.end);
  const LoopArgs a = loop_args(q, k, ld_qk, v, ld_v, g, beta, h0, Hk, Hv, scale, use_qk_l2norm, o, ht);
  return dt == GDN_BF16 ? dispatch<bf16>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream)
                        : dispatch<float>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream);
}

extern "C" size_t gdn_chunk_saved_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                                       int32_t dv, gdn_dtype dt) {
  (void)Hk;
  if (T < 0 || N < 0 || Hv < 1 || dk < 1 || dv < 1) return 0;
  return gdn::chunk_saved_layout(T, N, Hv, dk, dv, dt).end;
}

extern "C" int gdn_chunk_fwd_save(const void* q, const void* k, int64_t ld_qk, const void* v,
                                  int64_t ld_v, const float* g, const float* beta, const float* h0,
                                  const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                                  int32_t Hv, int32_t dk, int32_t dv, float scale,
                                  int use_qk_l2norm, void* o, float* ht, void* saved,
                                  size_t saved_bytes, void* ws, size_t ws_bytes, gdn_dtype dt,
                                  hipStream_t stream) {
  const char* fn = "gdn_chunk_fwd_save";
  int rc = gdn::validate_chunk(fn, q, k, ld_qk, v, ld_v, g, beta, cu_seqlens, N, T, Hk, Hv, dk, dv,
                               dt);
  if (rc != GDN_OK) return rc;
  if ((rc = check_out(fn, o, ht, N, T, cu_seqlens)) != GDN_OK) return rc;
  const Plan pl = fwd_plan(T, N, Hv, dk, dv, dt);
  if (!ws || ws_bytes < pl.end || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn, pl.end);
  const gdn::SavedLayout SL = gdn::chunk_saved_layout(T, N, Hv, dk, dv, dt);
  if (!saved || saved_bytes < SL.end || (reinterpret_cast<uintptr_t>(saved) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "%s: saved buffer needs %zu bytes, 256-byte aligned", fn,
                     SL.end);
  LoopArgs a = loop_args(q, k, ld_qk, v, ld_v, g, beta, h0, Hk, Hv, scale, use_qk_l2norm, o, ht);
  char* sv = static_cast<char*>(saved);
  a.states = sv + SL.off_states;
  char* rec = gdn::chunk_rec_bytes(dt) ? sv + SL.off_rec : nullptr;
  return dt == GDN_BF16 ? dispatch<bf16>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream, rec)
                        : dispatch<float>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream, rec);
}

extern "C" size_t gdn_chunk_fwd_gated_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                                     int32_t dk, int32_t dv, gdn_dtype dt) {
  (void)Hk;
  if (T < 0 || N < 0 || Hv < 1 || dk < 1 || dv < 1) return 0;
  return gdn::round_up(fwd_plan(T, N, Hv, dk, dv, dt).end, 256) + gated_extra(T, Hv, dt, dk, dv);
}

extern "C" int gdn_chunk_fwd_gated(const void* q, const void* k, int64_t ld_qk, const void* v,
                                   int64_t ld_v, const void* a_proj, const void* b_proj,
                                   int64_t ld_ab, const float* A_log, const float* dt_bias,
                                   const float* h0, const int32_t* cu_seqlens, int32_t N, int64_t T,
                                   int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                                   int use_qk_l2norm, void* o, float* ht, float* g_out,
                                   float* beta_out, void* ws, size_t ws_bytes, gdn_dtype dt,
                                   hipStream_t stream) {
  const char* fn = "gdn_chunk_fwd_gated";
  // the projections stand in for g and beta in the shared checks
  int rc = gdn::validate_chunk(fn, q, k, ld_qk, v, ld_v, (const float*)a_proj, (const float*)b_proj,
                               cu_seqlens, N, T, Hk, Hv, dk, dv, dt);
  if (rc != GDN_OK) return rc;
  if ((rc = check_out(fn, o, ht, N, T, cu_seqlens)) != GDN_OK) return rc;
  if (ld_ab < Hv) return gdn::fail(GDN_EINVAL, "%s: ld_ab smaller than Hv", fn);
  if (T > 0 && (!A_log || !dt_bias)) return gdn::fail(GDN_EINVAL, "%s: null A_log or dt_bias", fn);
  const Plan pl = fwd_plan(T, N, Hv, dk, dv, dt);
  const size_t need = gdn_chunk_fwd_gated_workspace_size(T, N, Hk, Hv, dk, dv, dt);
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn, need);
  LoopArgs a = loop_args(q, k, ld_qk, v, ld_v, nullptr, nullptr, h0, Hk, Hv, scale, use_qk_l2norm,
                         o, ht);
  if (prep_path(dt, dk, dv)) {
    // the prep forms each token's gates as it loads them
    a.ga = a_proj;
    a.gb = b_proj;
    a.ld_ab = ld_ab;
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.g_out = g_out;
    a.beta_out = beta_out;
  } else {
    // kernels that read given gates: form them first (into the caller's
    // g_out / beta_out, else the workspace)
    char* extra = (char*)ws + gdn::round_up(pl.end, 256);
    const size_t half = gdn::round_up(sizeof(float) * (size_t)T * Hv, 256);
    float* gb = g_out ? g_out : reinterpret_cast<float*>(extra);
    float* bb = beta_out ? beta_out : reinterpret_cast<float*>(extra + half);
    if ((rc = gdn::launch_gating_fwd(a_proj, b_proj, ld_ab, A_log, dt_bias, T, Hv, gb, bb, dt,
                                     stream)) != GDN_OK)
      return rc;
    a.g = gb;
    a.beta = bb;
  }
  return dt == GDN_BF16 ? dispatch<bf16>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream)
                        : dispatch<float>(dk, dv, a, cu_seqlens, N, T, pl, (char*)ws, stream);
}
