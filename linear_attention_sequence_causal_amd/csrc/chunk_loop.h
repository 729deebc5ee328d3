// chunk_loop.h -- the serial chunk loop of the chunked gated delta rule and
// the segment machinery around it.
//
// hyper-parallel "linear_attention_context_parallel.py":
// _run_prepared_gdn_chunks (per chunk: v_new = u - w S;
// o = (qh o e^G) S + P v_new; S <- e^{G_C} S + (kh o e^{G_C - G})^T v_new),
// with the chunk preparation of chunk_common.h, per sequence of cu_seqlens.
//
// A workgroup owns one (segment, value head): a run of whole 64-token chunks
// of one sequence, processed in order with the [dk, dv] fp32 state resident
// in registers (each wave holds 32 state columns as MFMA accumulator tiles,
// which feed the next products directly).  When there are too few
// (sequence, head) chains to fill the GPU, sequences are cut into segments
// and the page's affine state summaries make the segments independent
// (_compute_gdn_state_summary_from_prepared,
// _merge_gdn_prefix_state_summaries_torch, _apply_gdn_state_summary -- its
// context-parallel exchange, here between workgroups of one GPU):
//   plan     one workgroup lists segments and chunks (chunk_plan.h);
//   summary  every segment that is not the last of its sequence computes
//            X = [M | E] with S_out = M S_in + E, running its chunks on the
//            extended state [dk, dk+dv] from [I | 0] (M columns see u = 0);
//   scan     per (sequence, head, 16 state columns), fold the summaries from
//            the sequence's initial state: S_{p+1} = M_p S_p + E_p;
//   final    every segment runs its chunks from its initial state and either
//            writes o (and ht at the sequence end) or, for the backward,
//            stores the state entering every chunk.
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_common.h"
#include "chunk_plan.h"
#include "gdn_internal.h"

namespace gdn_chunk {
namespace {

enum Mode { kOut = 0, kSummary = 1, kStates = 2 };

struct LoopArgs {
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
  const int32_t* counts;
  const int32_t* seg_chunk0;
  float* seg_state;  // [seg_cap][Hv][DK][DK+DV] summaries
  float* seg_init;   // [seg_cap][Hv][DK][DV] initial states of non-first segments
  float* states;     // kStates: [chunk_cap][Hv][DK][DV] state entering each chunk
};

template <typename E, int DK, int DV, int MODE>
struct LoopCfg {
  typedef E O;  // operand type equals the activation type (bf16 or fp32)
  static constexpr bool HAS_Q = MODE == kOut;
  static constexpr int NSC = MODE == kSummary ? DK + DV : DV;  // state columns
  static constexpr int NW = NSC / 32;
  static constexpr int NT = NW * 64;
  typedef Smem<O, DK, DV, HAS_Q> SM;
  typedef Prefetch<E, DK, DV, NT, HAS_Q> PF;
};

template <typename E, int DK, int DV, int MODE>
__global__ __launch_bounds__((LoopCfg<E, DK, DV, MODE>::NT)) void chunk_loop_kernel(LoopArgs a) {
  typedef LoopCfg<E, DK, DV, MODE> CF;
  typedef typename CF::O O;
  typedef Mfma<O> M;
  constexpr int NW = CF::NW, NT = CF::NT;
  constexpr int KS = M::KSTEP;
  constexpr int NSK = DK / KS;  // contraction steps over dk
  constexpr int NSB = BT / KS;  // contraction steps over the chunk
  constexpr int DKT = DK / 16;  // state row tiles
  constexpr bool OUT = MODE == kOut;
  typedef typename CF::SM SM;
  __shared__ SM sm;

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= a.counts[0]) return;
  const int4 ent = a.seg_table[seg];
  if (MODE == kSummary && (ent.w & kLast)) return;
  const int n = ent.x;
  const int64_t tb = ent.y, te = ent.z;
  const int Hv = a.Hv;
  const int qa = h / (Hv / a.Hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = wave * 32;                        // first state column of this wave
  const bool mcol = MODE == kSummary && c0 < DK;   // wave holds columns of M (u = 0)
  const int vc0 = MODE == kSummary ? c0 - DK : c0; // value column of the wave's first column

  zero_upper<O, CF::HAS_Q, NT>(sm, tid);

  // state tiles S[mt][nt]: rows 16mt + 4(lane/16) + j, cols c0 + 16nt + lane%16
  floatx4 S[DKT][2];
  {
    const float* src = nullptr;
    if (MODE != kSummary) {
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
          else if (src) v = src[row * DV + col];
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
    stage<E, O, DK, DV, NT, CF::HAS_Q>(sm, pf, a.scale, a.use_l2norm, tid);
    if (c + 1 < nchunks) pf.load(qp, kp, a.ld_qk, vp, a.ld_v, gp, bp, Hv, tc + BT, te, tid);
    if constexpr (MODE == kStates) {
      // the state entering this chunk, for the backward
      float* dst = a.states + ((int64_t)(a.seg_chunk0[seg] + c) * Hv + h) * DK * DV;
#pragma unroll
      for (int mt = 0; mt < DKT; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            dst[(16 * mt + 4 * (lane >> 4) + j) * DV + c0 + 16 * nt + (lane & 15)] = S[mt][nt][j];
    }
    __syncthreads();
    gram_kk<O, DK, NW>(sm, wave, lane);
    __syncthreads();
    solve<O, DK, NW, CF::HAS_Q>(sm, wave, lane);  // P tiles too; ends with a barrier

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
      // o = e^G o (qh S) + P v_new, staged in LDS over v (free after the
      // barrier above) and written below as whole 16-byte row pieces
      O* so = sm.v;
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
          const float eg = sm.eg[rb + j];
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
          so[(rb + j) * SM::LDV + c0 + (lane & 15)] = from_f<O>(acc0[j]);
          so[(rb + j) * SM::LDV + c0 + 16 + (lane & 15)] = from_f<O>(acc1[j]);
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
        const typename M::frag kf = M::load_col(sm.k, SM::LDK, 16 * mt, s * KS, lane);
        M::mma(acc0, kf, vb[s][0]);
        M::mma(acc1, kf, vb[s][1]);
      }
      S[mt][0] = acc0;
      S[mt][1] = acc1;
    }

    if constexpr (OUT) {
      __syncthreads();  // staged o complete
      typedef typename Vec16<E>::type V16;
      constexpr int VE = Vec16<E>::N;
      constexpr int OPR = DV / VE;
      E* op = (E*)a.o + (int64_t)h * DV;
      for (int i = tid; i < BT * OPR; i += NT) {
        const int row = i / OPR, vi = i % OPR;
        const int64_t t = tc + row;
        if (t < te)
          *reinterpret_cast<V16*>(op + t * (int64_t)Hv * DV + vi * VE) =
              *reinterpret_cast<const V16*>(sm.v + row * SM::LDV + vi * VE);
      }
    }
  }

  // final state: ht (output) or the summary X = [M | E]
  float* dst = nullptr;
  int ld = DV;
  if (MODE == kSummary) {
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

// Scan over segment summaries (fp32): per (sequence, head, 16 columns).
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

// Plan, summaries + scan when segments split a sequence, then the final pass
// in `FINAL` mode (kOut or kStates).  `a` carries the caller's tensors.
template <typename E, int DK, int DV, int FINAL>
int run_pipeline(LoopArgs a, const int32_t* cu, int N, int64_t T, const Plan& pl, char* ws,
                 bool with_chunks, hipStream_t stream) {
  PlanPtrs pp = pl.ptrs(ws, with_chunks);
  a.seg_table = pp.table;
  a.counts = pp.counts;
  a.seg_chunk0 = pp.seg_chunk0;
  a.seg_state = pl.split ? reinterpret_cast<float*>(ws + pl.off_state) : nullptr;
  a.seg_init = pl.split ? reinterpret_cast<float*>(ws + pl.off_init) : nullptr;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, (int)pl.seg_len,
                     (int)pl.seg_cap, (int)pl.chunk_cap, pp);
  if (int rc = gdn::check_launch("chunk plan")) return rc;
  if (pl.split) {
    typedef LoopCfg<E, DK, DV, kSummary> CS;
    hipLaunchKernelGGL((chunk_loop_kernel<E, DK, DV, kSummary>), dim3((unsigned)pl.seg_cap, a.Hv),
                       dim3(CS::NT), 0, stream, a);
    if (int rc = gdn::check_launch("chunk summary")) return rc;
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV>), dim3(N, a.Hv, DV / 16), dim3(256), 0, stream,
                       a.seg_state, a.seg_init, a.h0, pp.seq_off, pp.seq_nseg, a.Hv);
    if (int rc = gdn::check_launch("chunk scan")) return rc;
  }
  typedef LoopCfg<E, DK, DV, FINAL> CO;
  hipLaunchKernelGGL((chunk_loop_kernel<E, DK, DV, FINAL>), dim3((unsigned)pl.seg_cap, a.Hv),
                     dim3(CO::NT), 0, stream, a);
  return gdn::check_launch("chunk loop");
}

}  // namespace
}  // namespace gdn_chunk
