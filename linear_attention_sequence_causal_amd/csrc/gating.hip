// gating.hip -- gdn_gating_fwd / gdn_gating_bwd: the gating step of the
// hyper-parallel page's CP wrappers (beta = sigmoid(b),
// g = -exp(A_log) * softplus(a + dt_bias)) and its reverse mode.  HBM-bound
// elementwise kernels; the per-head parameter gradients are reduced in a
// fixed order (per-block partial sums, then one pass over the blocks).
#include <hip/hip_runtime.h>

#include "gating.h"
#include "gdn_internal.h"

namespace {

using gdn_gate::beta_of;
using gdn_gate::g_of;
using gdn_gate::sigmoid;
using gdn_gate::softplus;

constexpr int kHeadLanes = 64;   // lanes over heads
constexpr int kTokLanes = 4;     // lanes over tokens
constexpr int kTokPerBlock = 256;

template <typename E>
__global__ __launch_bounds__(256) void gating_fwd_kernel(const E* __restrict__ a,
                                                         const E* __restrict__ b, int64_t ld,
                                                         const float* __restrict__ A_log,
                                                         const float* __restrict__ dt_bias,
                                                         int64_t T, int Hv, float* __restrict__ g,
                                                         float* __restrict__ beta) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * Hv) return;
  const int64_t t = i / Hv;
  const int h = (int)(i - t * Hv);
  g[i] = g_of(to_f(a[t * ld + h]), A_log[h], dt_bias[h]);
  beta[i] = beta_of(to_f(b[t * ld + h]));
}

// Block: kTokPerBlock tokens, threads (token lane tl, head lane hl).  da, db
// elementwise; per (block, head) partial sums of dA_log = sum dg * g and
// ddt_bias = sum da, over the block's tokens in a fixed order.
template <typename E>
__global__ __launch_bounds__(256) void gating_bwd_kernel(
    const E* __restrict__ a, const E* __restrict__ b, int64_t ld, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const float* __restrict__ dg, const float* __restrict__ dbeta,
    int64_t T, int Hv, E* __restrict__ da, E* __restrict__ db, int64_t ld_d,
    float* __restrict__ part) {
  __shared__ float sA[kTokLanes][kHeadLanes], sD[kTokLanes][kHeadLanes];
  const int hl = threadIdx.x % kHeadLanes, tl = threadIdx.x / kHeadLanes;
  const int64_t t0 = (int64_t)blockIdx.x * kTokPerBlock;
  const int64_t t1 = t0 + kTokPerBlock < T ? t0 + kTokPerBlock : T;
  for (int h0 = 0; h0 < Hv; h0 += kHeadLanes) {
    const int h = h0 + hl;
    float accA = 0.f, accD = 0.f;
    if (h < Hv) {
      const float e = __expf(A_log[h]), dtb = dt_bias[h];
      for (int64_t t = t0 + tl; t < t1; t += kTokLanes) {
        const float x = to_f(a[t * ld + h]) + dtb;
        const float sb = sigmoid(to_f(b[t * ld + h]));
        const float dgv = dg[t * Hv + h];
        const float dx = -dgv * e * sigmoid(x);
        da[t * ld_d + h] = from_f<E>(dx);
        db[t * ld_d + h] = from_f<E>(dbeta[t * Hv + h] * sb * (1.f - sb));
        accD += dx;
        accA += dgv * (-e * softplus(x));
      }
    }
    sA[tl][hl] = accA;
    sD[tl][hl] = accD;
    __syncthreads();
    if (tl == 0 && h < Hv) {
      float sa = 0.f, sd = 0.f;
#pragma unroll
      for (int j = 0; j < kTokLanes; j++) {
        sa += sA[j][hl];
        sd += sD[j][hl];
      }
      part[((int64_t)blockIdx.x * Hv + h) * 2] = sa;
      part[((int64_t)blockIdx.x * Hv + h) * 2 + 1] = sd;
    }
    __syncthreads();
  }
}

// dA_log[h], ddt_bias[h]: the blocks' partial sums added in block order.
__global__ __launch_bounds__(256) void gating_bwd_sum_kernel(const float* __restrict__ part,
                                                             int nblocks, int Hv,
                                                             float* __restrict__ dA_log,
                                                             float* __restrict__ ddt_bias) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= Hv) return;
  float sa = 0.f, sd = 0.f;
  for (int i = 0; i < nblocks; i++) {
    sa += part[((int64_t)i * Hv + h) * 2];
    sd += part[((int64_t)i * Hv + h) * 2 + 1];
  }
  if (dA_log) dA_log[h] = sa;
  if (ddt_bias) ddt_bias[h] = sd;
}

int validate(const char* fn, const void* a, const void* b, int64_t ld, const float* A_log,
             const float* dt_bias, int64_t T, int32_t Hv, gdn_dtype dt) {
  if (T < 0 || Hv < 1) return gdn::fail(GDN_EINVAL, "%s: need T >= 0 and Hv >= 1", fn);
  if (dt != GDN_F32 && dt != GDN_BF16) return gdn::fail(GDN_EINVAL, "%s: unknown dtype", fn);
  if (ld < Hv) return gdn::fail(GDN_EINVAL, "%s: ld_ab smaller than Hv", fn);
  if (T > 0 && (!a || !b || !A_log || !dt_bias)) return gdn::fail(GDN_EINVAL, "%s: null pointer", fn);
  return GDN_OK;
}

}  // namespace

namespace gdn {
// the gates formed into g, beta on `stream` (used by the gated chunk forward
// where its kernels read given gates)
int launch_gating_fwd(const void* a, const void* b, int64_t ld, const float* A_log,
                      const float* dt_bias, int64_t T, int32_t Hv, float* g, float* beta,
                      gdn_dtype dt, hipStream_t stream) {
  const int64_t n = T * Hv;
  if (n == 0) return GDN_OK;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dt == GDN_BF16)
    hipLaunchKernelGGL(gating_fwd_kernel<bf16>, grid, dim3(256), 0, stream, (const bf16*)a,
                       (const bf16*)b, ld, A_log, dt_bias, T, Hv, g, beta);
  else
    hipLaunchKernelGGL(gating_fwd_kernel<float>, grid, dim3(256), 0, stream, (const float*)a,
                       (const float*)b, ld, A_log, dt_bias, T, Hv, g, beta);
  return check_launch("gdn_gating_fwd");
}
}  // namespace gdn

extern "C" int gdn_gating_fwd(const void* a, const void* b, int64_t ld_ab, const float* A_log,
                              const float* dt_bias, int64_t T, int32_t Hv, float* g, float* beta,
                              gdn_dtype dt, hipStream_t stream) {
  int rc = validate("gdn_gating_fwd", a, b, ld_ab, A_log, dt_bias, T, Hv, dt);
  if (rc != GDN_OK) return rc;
  if (T > 0 && (!g || !beta)) return gdn::fail(GDN_EINVAL, "gdn_gating_fwd: null output");
  if (T * (int64_t)Hv > ((int64_t)1 << 40)) return gdn::fail(GDN_EINVAL, "gdn_gating_fwd: too large");
  return gdn::launch_gating_fwd(a, b, ld_ab, A_log, dt_bias, T, Hv, g, beta, dt, stream);
}

extern "C" size_t gdn_gating_bwd_workspace_size(int64_t T, int32_t Hv) {
  if (T <= 0 || Hv < 1) return 0;
  const int64_t nb = (T + kTokPerBlock - 1) / kTokPerBlock;
  return gdn::round_up((size_t)nb * (size_t)Hv * 2 * sizeof(float), 256);
}

extern "C" int gdn_gating_bwd(const void* a, const void* b, int64_t ld_ab, const float* A_log,
                              const float* dt_bias, const float* dg, const float* dbeta, int64_t T,
                              int32_t Hv, void* da, void* db, int64_t ld_dab, float* dA_log,
                              float* ddt_bias, void* ws, size_t ws_bytes, gdn_dtype dt,
                              hipStream_t stream) {
  int rc = validate("gdn_gating_bwd", a, b, ld_ab, A_log, dt_bias, T, Hv, dt);
  if (rc != GDN_OK) return rc;
  if (ld_dab < Hv) return gdn::fail(GDN_EINVAL, "gdn_gating_bwd: ld_dab smaller than Hv");
  if (T > 0 && (!dg || !dbeta || !da || !db))
    return gdn::fail(GDN_EINVAL, "gdn_gating_bwd: null pointer");
  const size_t need = gdn_gating_bwd_workspace_size(T, Hv);
  if (need > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
    return gdn::fail(GDN_EWORKSPACE, "gdn_gating_bwd: workspace needs %zu bytes, 256-byte aligned",
                     need);
  const int nb = (int)((T + kTokPerBlock - 1) / kTokPerBlock);
  float* part = (float*)ws;
  if (nb > 0) {
    if (dt == GDN_BF16)
      hipLaunchKernelGGL(gating_bwd_kernel<bf16>, dim3(nb), dim3(256), 0, stream, (const bf16*)a,
                         (const bf16*)b, ld_ab, A_log, dt_bias, dg, dbeta, T, Hv, (bf16*)da,
                         (bf16*)db, ld_dab, part);
    else
      hipLaunchKernelGGL(gating_bwd_kernel<float>, dim3(nb), dim3(256), 0, stream, (const float*)a,
                         (const float*)b, ld_ab, A_log, dt_bias, dg, dbeta, T, Hv, (float*)da,
                         (float*)db, ld_dab, part);
    if ((rc = gdn::check_launch("gdn_gating_bwd"))) return rc;
  }
  if (dA_log || ddt_bias) {
    hipLaunchKernelGGL(gating_bwd_sum_kernel, dim3((Hv + 255) / 256), dim3(256), 0, stream, part, nb,
                       Hv, dA_log, ddt_bias);
    return gdn::check_launch("gdn_gating_bwd(sum)");
  }
  return GDN_OK;
}
