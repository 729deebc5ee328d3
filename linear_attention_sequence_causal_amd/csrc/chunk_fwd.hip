// chunk_fwd.hip -- chunked gated delta rule, forward.
//
// hyper-parallel "linear_attention_context_parallel.py":
// _run_prepared_gdn_chunks (per chunk: v_new = u - w S;
// o = (qh o e^G) S + P v_new; S <- e^{G_C} S + (kh o e^{G_C - G})^T v_new),
// with the chunk preparation of chunk_common.h, per sequence of cu_seqlens.
//
// Work decomposition.  A workgroup owns one (segment, value head): a run of
// whole 64-token chunks of one sequence, processed in order with the
// [dk, dv] fp32 state resident in registers (each wave holds 32 state
// columns as MFMA accumulator tiles, which feed the next products directly).
// When there are too few (sequence, head) chains to fill the GPU, sequences
// are cut into segments and the page's affine state summaries make the
// segments independent (_compute_gdn_state_summary_from_prepared,
// _merge_gdn_prefix_state_summaries_torch, _apply_gdn_state_summary -- the
// context-parallel p2p/all-gather exchange, here between workgroups of one
// GPU):
//   1. plan     one workgroup lists the segments of every sequence;
//   2. summary  every segment that is not the last of its sequence computes
//               X = [M | E] with S_out = M S_in + E, by running its chunks on
//               the extended state [dk, dk+dv] from [I | 0] (M columns see
//               u = 0);
//   3. scan     per (sequence, head, 16 state columns), fold the summaries
//               from the sequence's initial state: S_{p+1} = M_p S_p + E_p;
//   4. output   every segment runs its chunks from its initial state and
//               writes o (and ht for the last segment of a sequence).
// Without segmentation only steps 1 and 4 run.
#include <hip/hip_runtime.h>
#include <stdlib.h>

#include "chunk_common.h"
#include "gdn_internal.h"

using namespace gdn_chunk;

namespace {

constexpr int kFirst = 1, kLast = 2;

struct FwdArgs {
  const void* q;
  const void* k;
  int64_t ld_qk;
  const void* v;
  int64_t ld_v;
  const float* g;
  const float* beta;
  const float* h0;
  int Hk, Hv;
  float scale;
  int use_l2norm;
  void* o;
  float* ht;
  const int4* seg_table;
  const int32_t* seg_count;
  float* seg_state;       // [NS][Hv][DK][DK+DV] summaries
  float* seg_init;        // [NS][Hv][DK][DV] initial states of non-first segments
};

// ---------------------------------------------------------------------------
// 1. plan
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int64_t T,
                                                   int seg_len, int cap, int4* __restrict__ table,
                                                   int32_t* __restrict__ count,
                                                   int32_t* __restrict__ seq_off,
                                                   int32_t* __restrict__ seq_nseg) {
  __shared__ int buf[256];
  const int t = threadIdx.x;
  int running = 0;
  for (int base = 0; base < N; base += 256) {
    const int n = base + t;
    int64_t s = 0, e = 0;
    int ns = 0;
    if (n < N) {
      s = cu[n];
      e = cu[n + 1];
      s = s < 0 ? 0 : (s > T ? T : s);
      e = e < s ? s : (e > T ? T : e);
      ns = (int)((e - s + seg_len - 1) / seg_len);
    }
    buf[t] = ns;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = t >= off ? buf[t - off] : 0;
      __syncthreads();
      buf[t] += add;
      __syncthreads();
    }
    const int off = running + buf[t] - ns;
    const int total = buf[255];
    __syncthreads();
    if (n < N) {
      seq_off[n] = off;
      seq_nseg[n] = ns;
      for (int p = 0; p < ns; p++) {
        if (off + p >= cap) break;
        const int64_t a = s + (int64_t)p * seg_len;
        const int64_t b = a + seg_len < e ? a + seg_len : e;
        table[off + p] = make_int4(n, (int)a, (int)b, (p == 0 ? kFirst : 0) | (p == ns - 1 ? kLast : 0));
      }
    }
    running += total;
  }
  if (t == 0) *count = running < cap ? running : cap;
}

// ---------------------------------------------------------------------------
// 2./4. chunk loop (summary or output)
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV, bool SUMMARY>
struct FwdCfg {
  typedef E O;  // operand type equals the activation type (bf16 or fp32)
  static constexpr int NSC = SUMMARY ? DK + DV : DV;  // state columns
  static constexpr int NW = NSC / 32;
  static constexpr int NT = NW * 64;
  typedef Smem<O, DK, DV, !SUMMARY> SM;
  typedef Prefetch<E, DK, DV, NT, !SUMMARY> PF;
};

template <typename E, int DK, int DV, bool SUMMARY>
__global__ __launch_bounds__((FwdCfg<E, DK, DV, SUMMARY>::NT)) void chunk_loop_kernel(FwdArgs a) {
  typedef FwdCfg<E, DK, DV, SUMMARY> CF;
  typedef typename CF::O O;
  typedef Mfma<O> M;
  constexpr int NW = CF::NW, NT = CF::NT;
  constexpr int KS = M::KSTEP;
  constexpr int NSK = DK / KS;  // contraction steps over dk
  constexpr int NSB = BT / KS;  // contraction steps over the chunk
  constexpr int DKT = DK / 16;  // state row tiles
  constexpr bool OUT = !SUMMARY;
  typedef typename CF::SM SM;
  __shared__ SM sm;

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= *a.seg_count) return;
  const int4 ent = a.seg_table[seg];
  if (SUMMARY && (ent.w & kLast)) return;
  const int n = ent.x;
  const int64_t tb = ent.y, te = ent.z;
  const int Hv = a.Hv;
  const int qa = h / (Hv / a.Hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = wave * 32;  // first state column of this wave
  const bool mcol = SUMMARY && c0 < DK;  // wave holds columns of M (u = 0)
  const int vc0 = SUMMARY ? c0 - DK : c0;  // value column of the wave's first column

  zero_upper<O, OUT, NT>(sm, tid);

  // state tiles S[mt][nt]: rows 16mt + 4(lane/16) + j, cols c0 + 16nt + lane%16
  floatx4 S[DKT][2];
  {
    const float* src = nullptr;
    int ld = DV;
    if (OUT) {
      if (!(ent.w & kFirst)) src = a.seg_init + ((int64_t)seg * Hv + h) * DK * DV;
      else if (a.h0) src = a.h0 + ((int64_t)n * Hv + h) * DK * DV;
    }
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int row = 16 * mt + 4 * (lane >> 4) + j, col = c0 + 16 * nt + (lane & 15);
          float v = 0.f;
          if (mcol) v = (row == col) ? 1.f : 0.f;
          else if (src) v = src[row * ld + col];
          S[mt][nt][j] = v;
        }
  }

  const E* qp = (const E*)a.q + (int64_t)qa * DK;
  const E* kp = (const E*)a.k + (int64_t)qa * DK;
  const E* vp = (const E*)a.v + (int64_t)h * DV;
  const float* gp = a.g + h;
  const float* bp = a.beta + h;
  typename CF::PF pf;
  const int nchunks = (int)((te - tb + BT - 1) / BT);
  if (nchunks > 0) pf.load(qp, kp, a.ld_qk, vp, a.ld_v, gp, bp, Hv, tb, te, tid);

  for (int c = 0; c < nchunks; c++) {
    const int64_t tc = tb + (int64_t)c * BT;
    __syncthreads();  // the previous chunk's LDS readers are done
    stage<E, O, DK, DV, NT, OUT>(sm, pf, a.scale, a.use_l2norm, tid);
    if (c + 1 < nchunks) pf.load(qp, kp, a.ld_qk, vp, a.ld_v, gp, bp, Hv, tc + BT, te, tid);
    __syncthreads();
    gram<O, DK, NW, OUT>(sm, wave, lane);
    __syncthreads();
    solve<NW>(sm, wave, lane);  // ends with a barrier

    floatx4 u[4][2];
    if (!mcol) compute_u<O>(sm, vc0, lane, u);
    compute_w<O, DK, NW>(sm, wave, lane);
    __syncthreads();

    // v_new = u - w S
    typename M::frag sb[NSK][2];
#pragma unroll
    for (int s = 0; s < NSK; s++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) sb[s][nt] = acc_as_b<O>(S, s, nt);
    floatx4 vn[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      floatx4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
      for (int s = 0; s < NSK; s++) {
        const typename M::frag wf = M::load(sm.w, SM::LDK, 16 * mt, s * KS, lane);
        M::mma(acc0, wf, sb[s][0]);
        M::mma(acc1, wf, sb[s][1]);
      }
      vn[mt][0] = mcol ? -acc0 : u[mt][0] - acc0;
      vn[mt][1] = mcol ? -acc1 : u[mt][1] - acc1;
    }

    const float GC = sm.G[BT - 1];
    if constexpr (OUT) {
      // o = e^G o (qh S) + P v_new, stored straight from the accumulators:
      // per store, 16 lanes write 32 contiguous bytes of one token row
      E* op = (E*)a.o + (int64_t)h * DV + c0 + (lane & 15);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        floatx4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int s = 0; s < NSK; s++) {
          const typename M::frag qf = M::load(sm.q, SM::LDK, 16 * mt, s * KS, lane);
          M::mma(acc0, qf, sb[s][0]);
          M::mma(acc1, qf, sb[s][1]);
        }
        const int rb = 16 * mt + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float eg = __expf(sm.G[rb + j]);
          acc0[j] *= eg;
          acc1[j] *= eg;
        }
#pragma unroll
        for (int s = 0; s < NSB; s++) {
          const typename M::frag pfrag = M::load(sm.p, SM::LDT, 16 * mt, s * KS, lane);
          M::mma(acc0, pfrag, acc_as_b<O>(vn, s, 0));
          M::mma(acc1, pfrag, acc_as_b<O>(vn, s, 1));
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int64_t t = tc + rb + j;
          if (t < te) {
            op[t * (int64_t)Hv * DV] = from_f<E>(acc0[j]);
            op[t * (int64_t)Hv * DV + 16] = from_f<E>(acc1[j]);
          }
        }
      }
    }

    // S <- e^{G_C} S + kh^T (e^{G_C - G} o v_new)
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const int rb = 16 * mt + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float d = __expf(GC - sm.G[rb + j]);
        vn[mt][0][j] *= d;
        vn[mt][1][j] *= d;
      }
    }
    const float eC = __expf(GC);
    typename M::frag vb[NSB][2];
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) vb[s][nt] = acc_as_b<O>(vn, s, nt);
#pragma unroll
    for (int mt = 0; mt < DKT; mt++) {
      floatx4 acc0 = S[mt][0] * eC, acc1 = S[mt][1] * eC;
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        const typename M::frag kf = M::load(sm.kt, SM::LDT, 16 * mt, s * KS, lane);
        M::mma(acc0, kf, vb[s][0]);
        M::mma(acc1, kf, vb[s][1]);
      }
      S[mt][0] = acc0;
      S[mt][1] = acc1;
    }

  }

  // final state: ht (output) or the summary X = [M | E]
  float* dst = nullptr;
  int ld = DV;
  if (SUMMARY) {
    dst = a.seg_state + ((int64_t)seg * Hv + h) * DK * (DK + DV);
    ld = DK + DV;
  } else if ((ent.w & kLast) && a.ht) {
    dst = a.ht + ((int64_t)n * Hv + h) * DK * DV;
  }
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int row = 16 * mt + 4 * (lane >> 4) + j, col = c0 + 16 * nt + (lane & 15);
          dst[row * ld + col] = S[mt][nt][j];
        }
  }
}

// ---------------------------------------------------------------------------
// 3. scan over segment summaries (fp32)
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ seg_state,
                                                       float* __restrict__ seg_init,
                                                       const float* __restrict__ h0,
                                                       const int32_t* __restrict__ seq_off,
                                                       const int32_t* __restrict__ seq_nseg, int Hv) {
  const int n = blockIdx.x, h = blockIdx.y, cb = blockIdx.z * 16;
  const int nseg = seq_nseg[n];
  if (nseg <= 1) return;
  const int off = seq_off[n];
  __shared__ float hs[DK][16];
  const int t = threadIdx.x, col = t & 15, r0 = t >> 4;
  for (int r = r0; r < DK; r += 16)
    hs[r][col] = h0 ? h0[(((int64_t)n * Hv + h) * DK + r) * DV + cb + col] : 0.f;
  __syncthreads();
  for (int p = 0; p + 1 < nseg; p++) {
    const float* X = seg_state + ((int64_t)(off + p) * Hv + h) * DK * (DK + DV);
    float nv[DK / 16];
#pragma unroll
    for (int i = 0; i < DK / 16; i++) {
      const int r = r0 + 16 * i;
      float acc = X[r * (DK + DV) + DK + cb + col];
      for (int m = 0; m < DK; m++) acc += X[r * (DK + DV) + m] * hs[m][col];
      nv[i] = acc;
    }
    __syncthreads();
    float* dst = seg_init + ((int64_t)(off + p + 1) * Hv + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < DK / 16; i++) {
      const int r = r0 + 16 * i;
      hs[r][col] = nv[i];
      dst[r * DV + cb + col] = nv[i];
    }
    __syncthreads();
  }
}

// ht of empty sequences = h0 (or zero).
__global__ __launch_bounds__(256) void empty_seq_state_kernel(const int32_t* __restrict__ cu,
                                                              const float* __restrict__ h0,
                                                              float* __restrict__ ht, int Hv,
                                                              int dd) {
  const int n = blockIdx.x, h = blockIdx.y;
  if (cu[n + 1] > cu[n]) return;
  const int64_t base = ((int64_t)n * Hv + h) * dd;
  for (int i = threadIdx.x; i < dd; i += 256) ht[base + i] = h0 ? h0[base + i] : 0.f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Plan {
  int64_t seg_len;
  int64_t cap;  // segment table capacity
  bool split;   // some sequence may have more than one segment
  size_t off_count, off_table, off_seq_off, off_seq_nseg, off_state, off_init, total;
};

Plan make_plan(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv) {
  Plan p{};
  const int64_t chunks = (T + BT - 1) / BT + N;  // bound on chunk count over all sequences
  int64_t per = 1;
  const char* env = getenv("GDN_SEG_CHUNKS");
  if (env && atoi(env) > 0) {
    per = atoi(env);
  } else {
    const int64_t cus = gdn::device_cu_count();
    per = (chunks * Hv + cus - 1) / cus;  // chunks per workgroup for one wave of the GPU
    if (per < 1) per = 1;
  }
  p.seg_len = per * BT;
  p.split = p.seg_len < T;
  p.cap = T / p.seg_len + N + 1;
  size_t o = 0;
  p.off_count = o;
  o = gdn::round_up(o + 4, 256);
  p.off_table = o;
  o = gdn::round_up(o + sizeof(int4) * (size_t)p.cap, 256);
  p.off_seq_off = o;
  o = gdn::round_up(o + 4 * (size_t)N, 256);
  p.off_seq_nseg = o;
  o = gdn::round_up(o + 4 * (size_t)N, 256);
  p.off_state = o;
  if (p.split) o = gdn::round_up(o + sizeof(float) * (size_t)p.cap * Hv * dk * (dk + dv), 256);
  p.off_init = o;
  if (p.split) o = gdn::round_up(o + sizeof(float) * (size_t)p.cap * Hv * dk * dv, 256);
  p.total = o;
  return p;
}

template <typename E, int DK, int DV>
int launch_fwd(const FwdArgs& base, const int32_t* cu, int N, int64_t T, const Plan& pl, char* ws,
               hipStream_t stream) {
  FwdArgs a = base;
  a.seg_table = reinterpret_cast<const int4*>(ws + pl.off_table);
  a.seg_count = reinterpret_cast<const int32_t*>(ws + pl.off_count);
  a.seg_state = pl.split ? reinterpret_cast<float*>(ws + pl.off_state) : nullptr;
  a.seg_init = pl.split ? reinterpret_cast<float*>(ws + pl.off_init) : nullptr;
  int32_t* seq_off = reinterpret_cast<int32_t*>(ws + pl.off_seq_off);
  int32_t* seq_nseg = reinterpret_cast<int32_t*>(ws + pl.off_seq_nseg);

  if (N > 0 && a.ht) {
    hipLaunchKernelGGL(empty_seq_state_kernel, dim3(N, a.Hv), dim3(256), 0, stream, cu, a.h0, a.ht,
                       a.Hv, DK * DV);
    if (int rc = gdn::check_launch("gdn_chunk_fwd(empty)")) return rc;
  }
  if (T == 0 || N == 0) return GDN_OK;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, (int)pl.seg_len,
                     (int)pl.cap, (int4*)a.seg_table, (int32_t*)a.seg_count, seq_off, seq_nseg);
  if (int rc = gdn::check_launch("gdn_chunk_fwd(plan)")) return rc;
  if (pl.split) {
    typedef FwdCfg<E, DK, DV, true> CS;
    hipLaunchKernelGGL((chunk_loop_kernel<E, DK, DV, true>), dim3((unsigned)pl.cap, a.Hv),
                       dim3(CS::NT), 0, stream, a);
    if (int rc = gdn::check_launch("gdn_chunk_fwd(summary)")) return rc;
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV>), dim3(N, a.Hv, DV / 16), dim3(256), 0, stream,
                       a.seg_state, a.seg_init, a.h0, seq_off, seq_nseg, a.Hv);
    if (int rc = gdn::check_launch("gdn_chunk_fwd(scan)")) return rc;
  }
  typedef FwdCfg<E, DK, DV, false> CO;
  hipLaunchKernelGGL((chunk_loop_kernel<E, DK, DV, false>), dim3((unsigned)pl.cap, a.Hv),
                     dim3(CO::NT), 0, stream, a);
  return gdn::check_launch("gdn_chunk_fwd");
}

template <typename E>
int dispatch(int dk, int dv, const FwdArgs& a, const int32_t* cu, int N, int64_t T, const Plan& pl,
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
// shared with the backward: argument validation of the chunk entry points
int validate_chunk(const char* fn, const void* q, const void* k, int64_t ld_qk, const void* v,
                   int64_t ld_v, const float* g, const float* beta, const int32_t* cu, int32_t N,
                   int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  if (T < 0 || N < 0) return fail(GDN_EINVAL, "%s: negative T or N", fn);
  if (T > INT32_MAX) return fail(GDN_EINVAL, "%s: T must be < 2^31", fn);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_EINVAL, "%s: need Hk >= 1 and Hv %% Hk == 0 (Hk=%d Hv=%d)", fn, Hk, Hv);
  if (dt != GDN_F32 && dt != GDN_BF16) return fail(GDN_EINVAL, "%s: unknown dtype", fn);
  if (!((dk == 32 || dk == 64 || dk == 128) && (dv == 32 || dv == 64 || dv == 128)))
    return fail(GDN_EUNSUPPORTED, "%s: dk=%d dv=%d not in {32,64,128}", fn, dk, dv);
  if (ld_qk < (int64_t)Hk * dk || ld_v < (int64_t)Hv * dv)
    return fail(GDN_EINVAL, "%s: row strides smaller than the head blocks", fn);
  const int es = dt == GDN_BF16 ? 2 : 4;
  if ((ld_qk * es) % 16 || (ld_v * es) % 16)
    return fail(GDN_EINVAL, "%s: row strides must be multiples of 16 bytes", fn);
  if (T > 0) {
    if (N < 1) return fail(GDN_EINVAL, "%s: T > 0 needs N >= 1 sequences", fn);
    if (!q || !k || !v || !g || !beta || !cu) return fail(GDN_EINVAL, "%s: null pointer", fn);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
      return fail(GDN_EINVAL, "%s: q, k, v must be 16-byte aligned", fn);
  }
  return GDN_OK;
}
}  // namespace gdn

extern "C" size_t gdn_chunk_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                           int32_t dk, int32_t dv, gdn_dtype dt, int bwd);

size_t gdn_chunk_fwd_workspace(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv) {
  if (T < 0 || N < 0 || Hv < 1) return 0;
  return make_plan(T, N, Hv, dk, dv).total;
}

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
  const Plan pl = make_plan(T, N, Hv, dk, dv);
  if (!ws || ws_bytes < pl.total || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "gdn_chunk_fwd: workspace needs %zu bytes, 256-byte aligned",
                     pl.total);
  FwdArgs a{};
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
