// chunk_loop.h -- the serial chunk loop of the chunked gated delta rule and
// the segment machinery around it.
//
// hyper-parallel "linear_attention_context_parallel.py":
// _run_prepared_gdn_chunks (per chunk: v_new = u - w S;
// o = (qh o e^G) S + P v_new; S <- e^{G_C} S + (kh o e^{G_C - G})^T v_new),
// per sequence of cu_seqlens.
//
// A workgroup owns one (segment, value head): a run of whole 64-token chunks
// of one sequence, processed in order with the [dk, dv] fp32 state resident
// in registers (each wave holds 32 state columns as MFMA accumulator tiles,
// which feed the next products directly).
//
// Per chunk the page forms u = T diag(beta) v and w = T diag(beta e^G) kh
// (T = (I + L)^-1) and then v_new = u - w S.  By linearity
//   v_new = T diag(beta) (v - diag(e^G) kh S),
// so each wave solves for its own state columns directly: kh S is one
// product, and T is applied by blocked forward substitution over the four
// 16-token block rows, x_i <- D_i (x_i - diag(beta_i) sum_{m<i} L_im x_m),
// with the inverted diagonal blocks D_i -- no T, u or w is ever formed and
// nothing of it passes through LDS.  q and k are staged raw; the l2norm and
// the q scale enter as per-row factors of the products.  When there are too few
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

#include <type_traits>

#include "chunk_common.h"
#include "chunk_plan.h"
#include "chunk_prep.h"
#include "gdn_internal.h"

namespace gdn_chunk {
namespace {

// kOutSave: the output mode that also stores the state entering every chunk
// (for a later backward), as kStates does.
enum Mode { kOut = 0, kSummary = 1, kStates = 2, kOutSave = 3 };
__host__ __device__ constexpr bool is_out(int mode) { return mode == kOut || mode == kOutSave; }
__host__ __device__ constexpr bool stores_states(int mode) { return mode == kStates || mode == kOutSave; }

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
  void* states;      // kStates, kOutSave: [chunk_cap][Hv][DK][DV] state entering each
                     // chunk, in the activation type (the backward uses it as MFMA
                     // operands of that type)
  const char* rec;   // prepared chunk records [chunk_cap][Hv] (bf16 state pass)
  int seg_cap;       // capacity of the segment table
  int seg_span;      // the state-pass grid covers segments 0 .. seg_span - 1
  int summary_all;         // kSummary: summarise a sequence's last segment too
  // replay (warm_kernel): per (segment, head) the chunks before the segment
  // that its final pass replays from a zero state (| kWarmFromStart: from
  // the sequence start, with h0); per (sequence, head) 1 when every segment
  // but the first replays, and then no summary or scan is needed.  Null:
  // summaries and scan as usual.
  const int32_t* warm;
  const int32_t* seq_warm;
  // gates formed from projections in the prep (ga non-null; bf16 prep
  // path), else the prep reads g, beta
  const void* ga;
  const void* gb;
  int64_t ld_ab;
  const float* A_log;
  const float* dt_bias;
  float* g_out;
  float* beta_out;
};

// The prep's view of a call's gates.
inline gdn_gate::Gates prep_gates(const LoopArgs& a) {
  return gdn_gate::Gates{a.g, a.beta, a.ga, a.gb, a.ld_ab, a.A_log, a.dt_bias, a.g_out, a.beta_out};
}

// LDS of the chunk loop (one chunk of one head at a time; rows padded by
// 16 bytes).  q, k are the raw rows (l2norm enters as per-row factors), v the
// raw values (later the staged output), p the decayed q k^T, L the strict
// lower kh kh^T o Gamma in fp32 whose diagonal 16x16 blocks are replaced by
// D_b = (I + diag(beta) L_bb)^-1.
template <typename O, int DK, int DV, bool HAS_Q>
struct LoopSmem {
  static constexpr int PAD = 16 / (int)sizeof(O);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDV = DV + PAD;
  static constexpr int LDP = BT + PAD;
  static constexpr int LDF = BT + 4;
  // small per-row arrays first: ds_read/ds_write immediate offsets reach
  // 64 KiB, so everything addressed per row stays within reach of one base
  alignas(16) float G[BT];
  alignas(16) float beta[BT];
  alignas(16) float eg[BT];  // exp(G)
  alignas(16) float rq[BT];  // scale / |q| (scale without l2norm)
  alignas(16) float rk[BT];  // 1 / |k| (1 without l2norm)
  alignas(16) float L[BT * LDF];
  alignas(16) O p[HAS_Q ? BT * LDP : 8];
  alignas(16) O k[BT * LDK];
  alignas(16) O q[HAS_Q ? BT * LDK : 8];
  alignas(16) O v[BT * LDV];
};

template <typename E, int DK, int DV, int MODE>
struct LoopCfg {
  typedef E O;  // operand type equals the activation type (bf16 or fp32)
  static constexpr bool HAS_Q = is_out(MODE);
  static constexpr int NSC = MODE == kSummary ? DK + DV : DV;  // state columns
  static constexpr int NW = NSC / 32;
  static constexpr int NT = NW * 64;
  typedef LoopSmem<O, DK, DV, HAS_Q> SM;
  typedef Prefetch<E, DK, DV, NT, HAS_Q> PF;
};

// Register prefetch -> LDS as raw rows, plus the per-row l2norm factors and
// the in-chunk cumsum of g.  Rows past the sequence end are zero.
template <typename E, int DK, int DV, int NT, bool HAS_Q, bool HAS_V, class SM>
GDN_DEV void stage_raw(SM& sm, const Prefetch<E, DK, DV, NT, HAS_Q, HAS_V>& pf, float scale,
                       int use_l2norm, int tid) {
  typedef Prefetch<E, DK, DV, NT, HAS_Q, HAS_V> PF;
  typedef typename Vec16<E>::type V16;
  constexpr int VE = PF::VE;
#pragma unroll
  for (int p = 0; p < PF::PQ; p++) {
    const int i = tid + NT * p;
    const int row = i / PF::QPR, vi = i % PF::QPR;
    float kss = sum_sq(pf.k[p]), qss = 0.f;
    if constexpr (HAS_Q) qss = sum_sq(pf.q[p]);
    if constexpr (PF::QPR <= 16) {
      kss = row_group_sum<PF::QPR>(kss);
      if constexpr (HAS_Q) qss = row_group_sum<PF::QPR>(qss);
    } else {
      kss = group_sum<PF::QPR>(kss);
      if constexpr (HAS_Q) qss = group_sum<PF::QPR>(qss);
    }
    if (i < PF::QV) {
      *reinterpret_cast<V16*>(sm.k + row * SM::LDK + vi * VE) = pf.k[p];
      if constexpr (HAS_Q) *reinterpret_cast<V16*>(sm.q + row * SM::LDK + vi * VE) = pf.q[p];
      if (vi == 0) {
        sm.rk[row] = use_l2norm ? __builtin_amdgcn_rsqf(kss + 1e-6f) : 1.f;
        if constexpr (HAS_Q) sm.rq[row] = use_l2norm ? scale * __builtin_amdgcn_rsqf(qss + 1e-6f) : scale;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PF::PV; p++) {
    const int i = tid + NT * p;
    const int row = i / PF::VPR, vi = i % PF::VPR;
    if (i < PF::VV) *reinterpret_cast<V16*>(sm.v + row * SM::LDV + vi * VE) = pf.v[p];
  }
  if (tid < BT) {  // wave 0: inclusive scan of g over the 64 rows
    float G = pf.g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(G, off, 64);
      if (tid >= off) G += o;
    }
    sm.G[tid] = G;
    sm.beta[tid] = pf.beta;
    sm.eg[tid] = __expf(G);
  }
}

// Lower 16x16 tile (i, j) of k k^T (-> L) or q k^T (-> P) from raw rows, with
// the l2norm factors and the decay exp(G_r - G_c).
template <typename O, int DK, class SM>
GDN_DEV void gram_tile_raw(SM& sm, bool isq, int i, int j, int lane) {
  typedef Mfma<O> M;
  floatx4 acc = zero4();
  const O* A = isq ? sm.q : sm.k;
#pragma unroll
  for (int s = 0; s < DK / M::KSTEP; s++)
    M::mma(acc, M::load(A, SM::LDK, 16 * i, s * M::KSTEP, lane),
           M::load(sm.k, SM::LDK, 16 * j, s * M::KSTEP, lane));
  const int col = 16 * j + (lane & 15);
  const int rb = 16 * i + 4 * (lane >> 4);
  const float Gc = sm.G[col], rc = sm.rk[col];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    const int row = rb + jj;
    const float dec = row >= col ? __expf(sm.G[row] - Gc) : 0.f;
    if (!isq) {
      sm.L[row * SM::LDF + col] = row > col ? acc[jj] * sm.rk[row] * rc * dec : 0.f;
    } else {
      sm.p[row * SM::LDP + col] = from_f<O>(acc[jj] * sm.rq[row] * rc * dec);
    }
  }
}

// Column j of D_b = (I + diag(beta_b) L_bb)^-1 by column-oriented forward
// substitution, written over L_bb.
template <class SM>
GDN_DEV void invert_diag_block(SM& sm, int b, int j) {
  constexpr int LDF = SM::LDF;
  float* Lb = sm.L + (16 * b) * LDF + 16 * b;
  const float* bb = sm.beta + 16 * b;
  // keep the unit vector's construction inside the chunk loop (hoisted, it
  // would pin 16 registers for the whole kernel)
  int jj;
  asm volatile("v_mov_b32 %0, %1" : "=v"(jj) : "v"(j));
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; i++) x[i] = (i == jj) ? 1.f : 0.f;
#pragma unroll
  for (int m = 0; m < 15; m++) {
#pragma unroll
    for (int i = m + 1; i < 16; i++) x[i] -= bb[i] * Lb[i * LDF + m] * x[m];
  }
#pragma unroll
  // Lanes of one wave run in lockstep: every read of the block above is
  // issued before these writes.
  for (int i = 0; i < 16; i++) Lb[i * LDF + j] = x[i];
}

template <typename E, int DK, int DV, int MODE>
__global__ __launch_bounds__((LoopCfg<E, DK, DV, MODE>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
void chunk_loop_kernel(LoopArgs a) {
  typedef LoopCfg<E, DK, DV, MODE> CF;
  typedef typename CF::O O;
  typedef Mfma<O> M;
  typedef Tile16<O> T16;
  constexpr int NW = CF::NW, NT = CF::NT;
  constexpr int KS = M::KSTEP;
  constexpr int NSK = DK / KS;  // contraction steps over dk
  constexpr int NSB = BT / KS;  // contraction steps over the chunk
  constexpr int DKT = DK / 16;  // state row tiles
  constexpr bool OUT = is_out(MODE);
  typedef typename CF::SM SM;
  __shared__ SM sm;

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= a.counts[0]) return;
  const int4 ent = a.seg_table[seg];
  if (MODE == kSummary && (ent.w & kLast) && !a.summary_all) return;
  // a replaying sequence needs no summaries
  if (MODE == kSummary && a.seq_warm && a.seq_warm[(int64_t)ent.x * a.Hv + h]) return;
  const int n = ent.x;
  const int64_t tb = ent.y, te = ent.z;
  const int Hv = a.Hv;
  const int qa = h / (Hv / a.Hk);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g4 = lane >> 4, ln = lane & 15;
  const int c0 = wave * 32;                        // first state column of this wave
  const bool mcol = MODE == kSummary && c0 < DK;   // wave holds columns of M (v = 0)
  const int vc0 = MODE == kSummary ? c0 - DK : c0; // value column of the wave's first column

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
          const int row = 16 * mt + 4 * g4 + j, col = c0 + 16 * nt + ln;
          float v = 0.f;
          if (mcol) v = (row == col) ? 1.f : 0.f;
          else if (src) v = src[row * DV + col];
          S[mt][nt][j] = v;
        }
  }
  // upper tiles of P stay zero
  if constexpr (OUT)
    for (int e = tid; e < BT * BT; e += NT) {
      const int r = e / BT, c = e % BT;
      if ((c >> 4) > (r >> 4)) sm.p[r * SM::LDP + c] = from_f<O>(0.f);
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
    // Lane-dependent addresses are rebuilt every chunk from an opaque copy of
    // the thread index: hoisted out of the loop they would pin dozens of
    // registers for its whole length.
    int tid_c = tid;
    asm volatile("" : "+v"(tid_c));
    const int lane = tid_c & 63, g4 = lane >> 4, ln = lane & 15;
    lds_barrier();  // the previous chunk's LDS readers are done
    stage_raw(sm, pf, a.scale, a.use_l2norm, tid_c);
    if constexpr (stores_states(MODE)) {
      // the state entering this chunk, for the backward
      E* dst = (E*)a.states + ((int64_t)(a.seg_chunk0[seg] + c) * Hv + h) * DK * DV;
#pragma unroll
      for (int mt = 0; mt < DKT; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            dst[(16 * mt + 4 * g4 + j) * DV + c0 + 16 * nt + ln] = from_f<E>(S[mt][nt][j]);
    }
    lds_barrier();
    // L (and P) tiles
    {
      constexpr int NTILE = OUT ? 20 : 10;
#pragma unroll 1
      for (int t = wave; t < NTILE; t += NW) {
        int i, j;
        lower_tile_ij(t % 10, i, j);
        gram_tile_raw<O, DK>(sm, t >= 10, i, j, lane);
      }
    }
    lds_barrier();
    // D_b = (I + diag(beta) L_bb)^-1, one 16-lane group per block
    if (NW >= 4) {
      if (wave < 4 && lane < 16) invert_diag_block(sm, wave, lane);
    } else if (wave == 0) {
      invert_diag_block(sm, g4, ln);
    }

    // (k S) for this wave's columns
    floatx4 x[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      floatx4 k0 = zero4(), k1 = zero4();
#pragma unroll
      for (int s = 0; s < NSK; s++) {
        const typename M::frag kf = M::load(sm.k, SM::LDK, 16 * mt, s * KS, lane);
        M::mma(k0, kf, acc_as_b<O>(S, s, 0));
        M::mma(k1, kf, acc_as_b<O>(S, s, 1));
      }
      // right-hand side beta o (v - exp(G) o (kh S))
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 16 * mt + 4 * g4 + j;
        const float bt = sm.beta[row], gk = sm.eg[row] * sm.rk[row];
        const float v0 = mcol ? 0.f : to_f(sm.v[row * SM::LDV + vc0 + ln]);
        const float v1 = mcol ? 0.f : to_f(sm.v[row * SM::LDV + vc0 + 16 + ln]);
        x[mt][0][j] = bt * (v0 - gk * k0[j]);
        x[mt][1][j] = bt * (v1 - gk * k1[j]);
      }
    }
    lds_barrier();  // D blocks written; v reads done
    // S's operand copy is rebuilt from the accumulators for (q S) below; kept
    // live through the solve it would cost 32 registers
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) asm volatile("" : "+v"(S[mt][nt]));

    // v_new = (I + diag(beta) L)^-1 rhs, block rows in order:
    // x_i <- D_i (x_i - diag(beta_i) sum_{m<i} L_im x_m)
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
      for (int m = 0; m < i; m++) {
        const float nb = -sm.beta[16 * i + ln];
        const typename T16::frag lf = T16::load_f32(sm.L, SM::LDF, 16 * i, 16 * m, nb, lane);
        T16::mma(x[i][0], lf, T16::from_acc(x[m][0]));
        T16::mma(x[i][1], lf, T16::from_acc(x[m][1]));
      }
      const typename T16::frag df = T16::load_f32(sm.L, SM::LDF, 16 * i, 16 * i, 1.f, lane);
      floatx4 y0 = zero4(), y1 = zero4();
      T16::mma(y0, df, T16::from_acc(x[i][0]));
      T16::mma(y1, df, T16::from_acc(x[i][1]));
      x[i][0] = y0;
      x[i][1] = y1;
    }

    const float GC = sm.G[BT - 1];
    if constexpr (OUT) {
      // o = (rq e^G) o (q S) + P v_new, staged over v, written below as whole
      // 16-byte row pieces
      O* so = sm.v;
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const int rb = 16 * mt + 4 * g4;
        floatx4 acc0 = zero4(), acc1 = zero4();
#pragma unroll
        for (int s = 0; s < NSK; s++) {
          const typename M::frag qf = M::load(sm.q, SM::LDK, 16 * mt, s * KS, lane);
          M::mma(acc0, qf, acc_as_b<O>(S, s, 0));
          M::mma(acc1, qf, acc_as_b<O>(S, s, 1));
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float f = sm.eg[rb + j] * sm.rq[rb + j];
          acc0[j] *= f;
          acc1[j] *= f;
        }
#pragma unroll
        for (int s = 0; s < NSB; s++) {
          const typename M::frag pfrag = M::load(sm.p, SM::LDP, 16 * mt, s * KS, lane);
          M::mma(acc0, pfrag, acc_as_b<O>(x, s, 0));
          M::mma(acc1, pfrag, acc_as_b<O>(x, s, 1));
        }
#pragma unroll
        for (int j = 0; j < 4; j++) {
          so[(rb + j) * SM::LDV + c0 + ln] = from_f<O>(acc0[j]);
          so[(rb + j) * SM::LDV + c0 + 16 + ln] = from_f<O>(acc1[j]);
        }
      }
    }

    // the next chunk's rows, in flight during the state update
    if (c + 1 < nchunks) pf.load(qp, kp, a.ld_qk, vp, a.ld_v, gp, bp, Hv, tc + BT, te, tid_c);

    // S <- e^{G_C} S + k^T (rk e^{G_C - G} o v_new)
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const int rb = 16 * mt + 4 * g4;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float d = sm.rk[rb + j] * __expf(GC - sm.G[rb + j]);
        x[mt][0][j] *= d;
        x[mt][1][j] *= d;
      }
    }
    const float eC = __expf(GC);
    typename M::frag vb[NSB][2];
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int nt = 0; nt < 2; nt++) vb[s][nt] = acc_as_b<O>(x, s, nt);
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
      lds_barrier();  // staged o complete
      typedef typename Vec16<E>::type V16;
      constexpr int VE = Vec16<E>::N;
      constexpr int OPR = DV / VE;
      E* op = (E*)a.o + (int64_t)h * DV;
      for (int i = tid_c; i < BT * OPR; i += NT) {
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
          const int row = 16 * mt + 4 * g4 + j, col = c0 + 16 * nt + ln;
          dst[row * ld + col] = S[mt][nt][j];
        }
  }
}

// ---------------------------------------------------------------------------
// State pass over prepared chunks (bf16 activations).
//
// chunk_prep.h has produced, for every (chunk, value head), the record of
// state-independent operators.  What is left per chunk is the chain through
// the state:
//   x = k S and o^T = S^T q^T (S's accumulators are the B, resp. A operands
//   directly),
//   x = T (v - fk o x)  (one lower-triangular product),
//   o^T = fo o o^T + x^T P^T  (stored from registers, four value columns of
//   one token per lane),
//   S <- eC S + k^T (fd o x)  (k^T read with the transposing LDS load).
// A workgroup owns one (segment, value head) and holds NC consumer waves, each
// owning 32 state columns as MFMA accumulator tiles, plus four loader waves
// that copy chunk c + 1 (rows of q, k, v and the record) into one of two LDS
// buffers while the consumers run chunk c from the other.  One workgroup
// barrier per chunk separates the two.

// The state's dk rows are kept permuted in registers: row r of accumulator
// tile mt holds dk = 32(mt/2) + 8(r/4) + 4(mt%2) + r%4.  Then the eight
// contraction elements a lane supplies to a 16x16x32 product (rows 4g..4g+3
// of tiles 2s and 2s+1) are dk 32s + 8g .. 32s + 8g + 7, contiguous in a k or
// q row: one 16-byte LDS read per fragment.
GDN_DEV int dk_of_row(int mt, int r) { return 32 * (mt >> 1) + 8 * (r >> 2) + 4 * (mt & 1) + (r & 3); }

// One LDS buffer: raw rows and the record.  Rows are padded by 32 bytes
// (288-byte rows for 128 bf16): the 16-byte row reads of q and k (rows
// l%16 of a fragment) then meet no bank conflict, and the transposing reads
// of k and v two-way ones (both measured with the SQ_LDS_BANK_CONFLICT
// counter on gfx950; 256- or 272-byte rows, or the 16-byte pieces of a row
// XOR-ed with a row bit, conflict on the row reads).
template <typename O, int DK, int DV, bool OUT>
struct WsSmem {
  static constexpr int PAD = 32 / (int)sizeof(O);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDV = DV + PAD;
  // bytes of the record the pass reads (G and rk only in the output pass)
  static constexpr int REC = OUT ? kRecEnd : kRecG;
  alignas(16) char rec[REC];
  alignas(16) char p[OUT ? 6 * 1024 : 16];  // P fragments, made by the loaders
  alignas(16) float fo[OUT ? 64 : 4];       // e^G rq
  alignas(16) float rq[OUT ? 64 : 4];       // l2norm factors of q (with the scale)
  alignas(16) O k[BT * LDK];
  alignas(16) O q[OUT ? BT * LDK : 8];
  alignas(16) O v[BT * LDV];
};

template <typename E, int DK, int DV, int MODE>
struct WsCfg {
  static constexpr bool OUT = is_out(MODE);
  static constexpr int NSC = MODE == kSummary ? DK + DV : DV;  // state columns
  // columns per consumer wave: 16 in the output pass (eight consumer waves, two
  // a SIMD, like the summary's), 32 otherwise
  static constexpr int CW = OUT && DV == 128 ? 16 : 32;
  static constexpr int NC = NSC / CW;                          // consumer waves
  static constexpr int NL = 4;                                 // loader waves
  static constexpr int NT = (NC + NL) * 64;
  typedef WsSmem<E, DK, DV, OUT> SM;
  static constexpr bool FITS = 2 * sizeof(SM) <= 160 * 1024;
};

// Buffer resource over `bytes` bytes from `base` (raw, stride 0): loads at
// offsets past the end return zero, so rows past a sequence end need no
// predicate and nothing outside the range is ever read.
GDN_DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename V>
GDN_DEV V buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// 8-byte store; past the end of the range it is dropped
template <typename V>
GDN_DEV void buffer_store8(const V& v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, 0);
}
// one element (2 or 4 bytes)
template <typename E>
GDN_DEV void buffer_store_elem(E v, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(E) == 2)
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, voff, soff, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, voff, soff, 0);
}

// Fragments of a 64 x 64 upper-triangular operator (P^T, T^T) as A operands
// that are not entirely below the diagonal: (row block mt, contraction half
// s) -> index, for (0,0) (0,1) (1,0) (1,1) (2,1) (3,1).
__host__ __device__ constexpr int pt_frag(int mt, int s) { return mt < 2 ? 2 * mt + s : mt + 2; }

// One 16-byte vector i (< 384) of a record's T fragments, element e of lane l
// of fragment p_frag(mt, s) = i / 64 being T[16 mt + l%16][32 s + 16 (e/4) +
// 4 (l/16) + e%4], written to LDS (dst) at its place in the fragments of T^T
// (the same convention, pt_frag order): the lower fragments of T fill the
// upper ones of T^T exactly.
GDN_DEV void store_t_transposed(char* dst, int i, const floatx4& v) {
  const bf16x8 t = __builtin_bit_cast(bf16x8, v);
  const int fp = i >> 6, l = i & 63;
  const int mt = fp < 2 ? fp : (fp + 2) >> 1, s = fp < 2 ? 0 : (fp & 1);
  const int g = l >> 4, ln = l & 15;
  // row r = 16 mt + ln of T is column r of T^T: contraction half s' = mt / 2,
  // lane group (r % 16) / 4, element 4 (mt % 2) + r % 4
  const int ep = 4 * (mt & 1) + (ln & 3);
#pragma unroll
  for (int e = 0; e < 8; e++) {
    // column c = 32 s + 16 (e/4) + 4 g + e%4 of T is row c of T^T
    const int mtp = 2 * s + (e >> 2), lanep = 16 * (ln >> 2) + 4 * g + (e & 3);
    *reinterpret_cast<bf16*>(dst + pt_frag(mtp, mt >> 1) * 1024 + lanep * 16 + ep * 2) = t[e];
  }
}

// Loader registers: one chunk's rows and the first RECB bytes of its record,
// 16-byte vectors.  The loads go through buffer resources
// based at the chunk's first row, so a thread's byte offsets are the same for
// every chunk (made once by `offsets`) and the per-chunk address work is
// scalar.
template <typename E, int DK, int DV, bool HAS_Q, int RECB>
struct WsLoad {
  typedef typename Vec16<E>::type V16;
  static constexpr int NTL = 256;  // loader threads
  static constexpr int VE = Vec16<E>::N;
  static constexpr int QPR = DK / VE, VPR = DV / VE;
  static constexpr int PQ = BT * QPR / NTL, PV = BT * VPR / NTL;
  static constexpr int RV = RECB / 16;  // record vectors
  static constexpr int PR = (RV + NTL - 1) / NTL;
  static_assert(BT * QPR % NTL == 0 && BT * VPR % NTL == 0 && RECB % 16 == 0, "loader split");
  static_assert(QPR <= 16 && NTL % QPR == 0, "a q row within one 16-lane group");
  V16 q[HAS_Q ? PQ : 1], k[PQ], v[PV];
  floatx4 r[PR];

  // this thread's byte offsets within a chunk (row tid / QPR, piece tid % QPR,
  // then NTL / QPR rows further per step p)
  struct Off {
    uint32_t qk, v, qk_step, v_step;
  };
  GDN_DEV static Off offsets(int64_t ld_qk, int64_t ld_v, int tid) {
    Off o;
    o.qk = (uint32_t)((tid / QPR) * ld_qk * (int64_t)sizeof(E) + (tid % QPR) * 16);
    o.v = (uint32_t)((tid / VPR) * ld_v * (int64_t)sizeof(E) + (tid % VPR) * 16);
    o.qk_step = (uint32_t)((NTL / QPR) * ld_qk * (int64_t)sizeof(E));
    o.v_step = (uint32_t)((NTL / VPR) * ld_v * (int64_t)sizeof(E));
    return o;
  }

  GDN_DEV void load(const E* qp, const E* kp, int64_t ld_qk, const E* vp, int64_t ld_v,
                    const char* rec, int64_t tc, int64_t te, const Off& off, int tid) {
    const int64_t rows = te - tc < BT ? te - tc : BT;  // rows of the chunk in its sequence (>= 1)
    // the last valid row ends its head slice inside the range; row `rows` starts past it
    const uint32_t qk_bytes = (uint32_t)(((rows - 1) * ld_qk + DK) * (int64_t)sizeof(E));
    const uint32_t v_bytes = (uint32_t)(((rows - 1) * ld_v + DV) * (int64_t)sizeof(E));
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kp + tc * ld_qk, qk_bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vp + tc * ld_v, v_bytes);
#pragma unroll
    for (int p = 0; p < PQ; p++) {
      if constexpr (HAS_Q) q[p] = buffer_load16<V16>(buffer_rsrc(qp + tc * ld_qk, qk_bytes), off.qk, p * off.qk_step);
      k[p] = buffer_load16<V16>(rk, off.qk, p * off.qk_step);
    }
#pragma unroll
    for (int p = 0; p < PV; p++) v[p] = buffer_load16<V16>(rv, off.v, p * off.v_step);
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(rec, (uint32_t)RECB);
#pragma unroll
    for (int p = 0; p < PR; p++) r[p] = buffer_load16<floatx4>(rr, 16u * tid, 16u * NTL * p);
  }
  // rows into LDS; with q, also its l2norm factors
  // (with the scale): a q row is QPR consecutive lanes.  T_TRANSPOSED: the
  // record's T fragments go to LDS as the fragments of T^T (see
  // store_t_transposed), the rest of the record as it is.
  template <bool T_TRANSPOSED = false, class SM>
  GDN_DEV void store(SM& sm, int tid, float scale, int use_l2norm) const {
#pragma unroll
    for (int p = 0; p < PQ; p++) {
      const int i = tid + NTL * p;
      const int row = i / QPR, vi = i % QPR;
      const int vx = vi;
      if constexpr (HAS_Q) {
        *reinterpret_cast<V16*>(sm.q + row * SM::LDK + vx * VE) = q[p];
        const float ss = row_group_sum<QPR>(sum_sq(q[p]));
        if (vi == 0) sm.rq[row] = use_l2norm ? scale * __builtin_amdgcn_rsqf(ss + 1e-6f) : scale;
      }
      *reinterpret_cast<V16*>(sm.k + row * SM::LDK + vx * VE) = k[p];
    }
#pragma unroll
    for (int p = 0; p < PV; p++) {
      const int i = tid + NTL * p;
      const int row = i / VPR, vi = i % VPR;
      *reinterpret_cast<V16*>(sm.v + row * SM::LDV + vi * VE) = v[p];
    }
#pragma unroll
    for (int p = 0; p < PR; p++) {
      const int i = tid + NTL * p;
      if (T_TRANSPOSED && i < 6 * 64)
        store_t_transposed(sm.rec + kRecT, i, r[p]);
      else if (i < RV)
        *reinterpret_cast<floatx4*>(sm.rec + 16 * i) = r[p];
    }
  }
};

// Hand-off among the loader waves through an LDS counter, without a
// workgroup barrier: each wave adds one when its rows are stored (arrive) and
// waits until `target` (NL a chunk so far) is reached.  Every loader wave
// runs the same iterations, so the wait ends.
GDN_DEV void count_arrive(unsigned* count, int lane) {
  wave_lds_sync();  // this wave's stores are done
  if (lane == 0) __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
GDN_DEV void count_wait(unsigned* count, unsigned target) {
  while (__hip_atomic_load(count, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
}

// The decayed q k^T of one chunk as the P fragments of the output product:
// element (tok, tok') = rq_tok rk_tok' e^{G_tok - G_tok'} q_tok . k_tok' for
// tok' <= tok.  Fragment (mt, s) holds in lane l row tok = 16 mt + l%16 and
// in its half h (elements 4h .. 4h + 3) the columns tok' = 32 s + 16 h +
// 4(l/16) + e: exactly the accumulator of the tile k_{j'} q_mt^T, j' = 2s + h.
// The twelve halves are dealt to the waves that make them in this order (the
// two that lie above the diagonal, all zero, last but two).
constexpr int kPHalves = 12;
__host__ __device__ constexpr int p_half_mt(int u) { return u < 8 ? (u < 4 ? (u == 0 ? 0 : u == 2 ? 1 : 2) : 3) : (u == 8 ? 0 : u == 10 ? 1 : 2); }
__host__ __device__ constexpr int p_half_s(int u) { return u == 1 || u == 6 || u == 7 || u == 9 ? 1 : 0; }
__host__ __device__ constexpr int p_half_h(int u) { return u == 5 || u == 7 || u >= 8 ? 1 : 0; }

// One half of P being made: begin() reads the operands and issues the
// products (no branches, so they interleave with the caller's next
// products), finish() scales, masks and stores.
template <int DK>
struct PHalf {
  int mt, s, h, jp;
  floatx4 acc;
  template <class SM>
  GDN_DEV void begin(const SM& C, int u, int lane, bool real) {
    mt = p_half_mt(u);
    s = p_half_s(u);
    h = p_half_h(u);
    jp = 2 * s + h;
    acc = zero4();
    if (real) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ks++)
        Mfma<bf16>::mma(acc, Mfma<bf16>::load_k8(C.k, SM::LDK, 16 * jp, 32 * ks, lane),
                        Mfma<bf16>::load_k8(C.q, SM::LDK, 16 * mt, 32 * ks, lane));
    }
  }
  template <class SM>
  GDN_DEV void finish(SM& C, int lane) const {
    const int g4 = lane >> 4, ln = lane & 15;
    const float* Gv = reinterpret_cast<const float*>(C.rec + kRecG);
    const int tok = 16 * mt + ln, tp0 = 16 * jp + 4 * g4;
    const float rqt = C.rq[tok], Gt = Gv[tok];
    const floatx4 rk4 = *reinterpret_cast<const floatx4*>(Gv + 64 + tp0);
    const floatx4 G4 = *reinterpret_cast<const floatx4*>(Gv + tp0);
    bf16x4 f;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float val = acc[e] * rqt * rk4[e] * __expf(fminf(Gt - G4[e], 0.f));
      f[e] = (bf16)(tp0 + e <= tok ? val : 0.f);
    }
    *reinterpret_cast<bf16x4*>(C.p + p_frag(mt, s) * 1024 + lane * 16 + h * 8) = f;
  }
};

// log of a transition norm below which a summary's M columns are zero
// (e^-200 is about 1e-87)
constexpr float kNegligibleLog = -200.f;

// Replay instead of summaries.  The state entering a segment is S = M_W S' +
// E_W over the W chunks before it, S' the state W chunks earlier.  When the
// records' bound on log |M_W| (the sum of their lb) is below kNegligibleLog,
// M_W S' is below 1e-87 |S'|: the state is E_W, the recurrence over those W
// chunks from zero, to far below the resolution of fp32.  A segment's final
// pass then replays those chunks itself (or, reaching the sequence start,
// runs from h0 exactly), and the sequence needs no summaries or scan.
constexpr int kWarmMax = 16;                 // longest replay tried, chunks
constexpr int32_t kWarmFromStart = 1 << 30;  // replay from the sequence start

// Per (sequence, head): the replay length of every segment but the first,
// -1 when the bound is not reached within kWarmMax chunks; seq_warm = 1 when
// none is -1.
__global__ __launch_bounds__(256) void warm_kernel(const char* __restrict__ rec, int Hv,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ seg_chunk0,
                                                   const int32_t* __restrict__ seq_off,
                                                   const int32_t* __restrict__ seq_nseg,
                                                   const int32_t* __restrict__ seq_chunk_off,
                                                   int seg_cap, int32_t* __restrict__ warm,
                                                   int32_t* __restrict__ seq_warm) {
  const int n = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int off = seq_off[n], nseg = seq_nseg[n], c0 = seq_chunk_off[n];
  const int nchunks = counts[1];
  int cold = 0;
  for (int p = 1 + t; p < nseg; p += 256) {
    const int s = off + p;
    if (s >= seg_cap) break;
    const int cb = seg_chunk0[s];
    int val = -1;
    float sum = 0.f;
    for (int w = 0; w < kWarmMax; w++) {
      const int c = cb - 1 - w;
      if (c < c0) {  // the sequence start: replay all of it, from h0
        val = w | kWarmFromStart;
        break;
      }
      if (c >= nchunks) break;
      sum += *reinterpret_cast<const float*>(rec + ((int64_t)c * Hv + h) * kRecBytes + kRecF +
                                             129 * sizeof(float));
      if (sum < kNegligibleLog) {
        val = w + 1;
        break;
      }
    }
    warm[(int64_t)s * Hv + h] = val;
    cold |= val < 0;
  }
  cold = __syncthreads_or(cold);
  if (t == 0) seq_warm[(int64_t)n * Hv + h] = cold ? 0 : 1;
}

// One (segment, value head) of the state pass in mode MODE, from LDS buffers
// `buf` and the P hand-off counter (zeroed).
template <typename E, int DK, int DV, int MODE>
GDN_DEV void ws_body(const LoopArgs& a, typename WsCfg<E, DK, DV, MODE>::SM* buf, unsigned* p_count_ptr,
                     int seg, int h, int4 ent) {
  typedef WsCfg<E, DK, DV, MODE> CF;
  typedef E O;
  typedef Mfma<O> M;
  typedef typename M::frag Fr;
  constexpr int NC = CF::NC;
  constexpr int NL = CF::NL;
  constexpr int CW = CF::CW;
  constexpr int NN = CW / 16;   // 16-column tiles per consumer wave
  constexpr int KS = M::KSTEP;  // 32
  constexpr int NSK = DK / KS;  // contraction steps over dk
  constexpr int NSB = BT / KS;  // contraction steps over the chunk
  constexpr int DKT = DK / 16;  // state row tiles
  constexpr bool OUT = CF::OUT;
  typedef typename CF::SM SM;
  static_assert(KS == 32, "bf16 fragments");
  unsigned& p_count = *p_count_ptr;
  const int n = ent.x;
  const int64_t tb = ent.y, te = ent.z;
  const int Hv = a.Hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g4 = lane >> 4, ln = lane & 15;
  const int nchunks = (int)((te - tb + BT - 1) / BT);
  const int chunk0 = a.seg_chunk0[seg];
  const char* recs = a.rec + (int64_t)h * kRecBytes;  // + chunk * Hv * kRecBytes
  // final passes of a replaying sequence: the chunks before the segment run
  // first (no outputs), from zero or, reaching the sequence start, from h0
  int nwarm = 0;
  bool warm_h0 = false;
  if (MODE != kSummary && a.seq_warm && !(ent.w & kFirst) && a.seq_warm[(int64_t)n * Hv + h]) {
    const int v = a.warm[(int64_t)seg * Hv + h];
    nwarm = v & ~kWarmFromStart;
    warm_h0 = (v & kWarmFromStart) != 0;
  }

  if (wave >= NC) {
    // ======================= loaders =======================
    typedef WsLoad<E, DK, DV, OUT, SM::REC> LD;
    const int ltid = tid - NC * 64;
    const int qa = h / (Hv / a.Hk);
    const E* qp = (const E*)a.q + (int64_t)qa * DK;
    const E* kp = (const E*)a.k + (int64_t)qa * DK;
    const E* vp = (const E*)a.v + (int64_t)h * DV;
    const int64_t rstride = (int64_t)Hv * kRecBytes;
    const typename LD::Off off = LD::offsets(a.ld_qk, a.ld_v, ltid);
    LD ld;
    // segment chunk pc (from -nwarm: the replayed ones) goes to buffer pc & 1
    if (nchunks > 0)
      ld.load(qp, kp, a.ld_qk, vp, a.ld_v, recs + (int64_t)(chunk0 - nwarm) * rstride,
              tb - (int64_t)nwarm * BT, te, off, ltid);
    for (int it = -1 - nwarm; it < nchunks; it++) {
      const int pc = it + 1;
      if (pc < nchunks) {
        SM& B = buf[pc & 1];
        ld.store(B, ltid, a.scale, a.use_l2norm);
        if (pc + 1 < nchunks)
          ld.load(qp, kp, a.ld_qk, vp, a.ld_v, recs + (int64_t)(chunk0 + pc + 1) * rstride,
                  tb + (int64_t)(pc + 1) * BT, te, off, ltid);
        if constexpr (OUT) {
          // P and fo of the chunk just stored, made here while the consumers
          // run the previous chunk: once every loader wave's rows are in
          // place (LDS counter among the loader waves), each makes its
          // three halves of P (all products issued before any is finished)
          const int lw = wave - NC;
          count_arrive(&p_count, lane);
          count_wait(&p_count, (unsigned)NL * (unsigned)(pc + nwarm + 1));
          constexpr int NR = kPHalves / NL;
          PHalf<DK> ph[NR];
#pragma unroll
          for (int r = 0; r < NR; r++) {
            const int u = lw + r * NL;
            ph[r].begin(B, u, lane, p_half_s(u) * 2 + p_half_h(u) <= p_half_mt(u));
          }
#pragma unroll
          for (int r = 0; r < NR; r++) ph[r].finish(B, lane);
          if (lw == 0) B.fo[lane] = __expf(reinterpret_cast<const float*>(B.rec + kRecG)[lane]) * B.rq[lane];
        }
      }
      lds_barrier();  // the chunk (with P and fo) is published
    }
    return;
  }

  // ======================= consumers =======================
  const int c0 = wave * CW;                         // first state column of this wave
  const bool mcol = MODE == kSummary && c0 < DK;    // wave holds columns of M (v = 0)
  const int vc0 = MODE == kSummary ? c0 - DK : c0;  // value column of the first column
  // state tiles S[mt][nt]: rows 16mt + 4(lane/16) + j, cols c0 + 16nt + lane%16
  floatx4 S[DKT][NN];
  {
    const float* src = nullptr;
    if (MODE != kSummary) {
      const float* h0n = a.h0 ? a.h0 + ((int64_t)n * Hv + h) * DK * DV : nullptr;
      if (nwarm > 0) src = warm_h0 ? h0n : nullptr;
      else if (!(ent.w & kFirst)) src = a.seg_init + ((int64_t)seg * Hv + h) * DK * DV;
      else src = h0n;
    }
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int row = dk_of_row(mt, 4 * g4 + j), col = c0 + 16 * nt + ln;
          float v = 0.f;
          if (mcol) v = (row == col) ? 1.f : 0.f;
          else if (src) v = src[row * DV + col];
          S[mt][nt][j] = v;
        }
  }
  const int64_t o_ld = (int64_t)Hv * DV;
  floatx4 x[4][NN], o[OUT ? 4 : 1][NN];
  // M columns of a summary: once the bound on the log of the transition's
  // norm accumulated over the segment (the records' lb) is below
  // kNegligibleLog, |M| < e^kNegligibleLog, far below the smallest bf16 or
  // fp32 magnitude: M is zero from there on and its waves skip their products
  float log_norm = 0.f;
  bool m_zero = false;
  // one chunk (buffer C, chunk it of the segment); EMIT false: a replayed
  // chunk, the state update only
  auto step = [&](auto emit, SM& C, const int it) {
    constexpr bool EMIT = decltype(emit)::value;
      const char* R = C.rec;
      if constexpr (stores_states(MODE) && EMIT) {
        // the state entering this chunk, for the backward: element stores
        // through a buffer resource over it, the lane's part of the offset
        // (row 8 g4 of dk_of_row, its column) fixed and the rest constant,
        // so the addresses take no registers
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc((E*)a.states + ((int64_t)(chunk0 + it) * Hv + h) * DK * DV,
                        (uint32_t)(DK * DV * sizeof(E)));
        const uint32_t soff = (uint32_t)((8 * g4 * DV + c0 + ln) * sizeof(E));
#pragma unroll
        for (int mt = 0; mt < DKT; mt++)
#pragma unroll
          for (int nt = 0; nt < NN; nt++)
#pragma unroll
            for (int j = 0; j < 4; j++)
              buffer_store_elem<E>(from_f<E>(S[mt][nt][j]), rs, soff,
                                   (uint32_t)(((32 * (mt >> 1) + 4 * (mt & 1) + j) * DV + 16 * nt) * sizeof(E)));
      }
      // k S (into x) and q S (into o), one contraction step of S at a time
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++) {
          x[mt][nt] = zero4();
          if constexpr (OUT && EMIT) o[mt][nt] = zero4();
        }
#pragma unroll
      for (int s = 0; s < NSK; s++) {
        Fr b[NN];
#pragma unroll
        for (int nt = 0; nt < NN; nt++) b[nt] = acc_as_b<O>(S, s, nt);
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          const Fr kf = M::load_k8(C.k, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
          for (int nt = 0; nt < NN; nt++) M::mma(x[mt][nt], kf, b[nt]);
          if constexpr (OUT && EMIT) {
            // o^T = S^T q^T: the state fragment is the A operand (its column
            // index is the row of the product), q rows the B operand
            const Fr qf = M::load_k8(C.q, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
            for (int nt = 0; nt < NN; nt++) M::mma(o[mt][nt], b[nt], qf);
          }
        }
      }
      const float* Fd = reinterpret_cast<const float*>(R + kRecF);
      const float* Fk = Fd + 64;
      const float eC = Fd[128];
      if (mcol) log_norm += Fd[129];
      // x = T (v - fk o (k S)): the right side in accumulator layout (token
      // rows), then one lower-triangular product with T's fragments
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const floatx4 f = *reinterpret_cast<const floatx4*>(Fk + 16 * i + 4 * g4);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) {
          floatx4 y = -f * x[i][nt];
          if (!mcol) {
            const bf16x4 vv = lds_rows4_tr(C.v, SM::LDV, 16 * i, vc0 + 16 * nt, lane);
#pragma unroll
            for (int j = 0; j < 4; j++) y[j] += (float)vv[j];
          }
          x[i][nt] = y;
        }
      }
      {
        Fr ys[NSB][NN];
#pragma unroll
        for (int s = 0; s < NSB; s++)
#pragma unroll
          for (int nt = 0; nt < NN; nt++) ys[s][nt] = acc_as_b<O>(x, s, nt);
#pragma unroll
        for (int mt = 0; mt < 4; mt++)
#pragma unroll
          for (int nt = 0; nt < NN; nt++) x[mt][nt] = zero4();
#pragma unroll
        for (int s = 0; s < NSB; s++)
#pragma unroll
          for (int mt = 2 * s; mt < 4; mt++) {
            const Fr tf = *reinterpret_cast<const Fr*>(R + kRecT + p_frag(mt, s) * 1024 + lane * 16);
#pragma unroll
            for (int nt = 0; nt < NN; nt++) M::mma(x[mt][nt], tf, ys[s][nt]);
          }
      }
      if constexpr (OUT && EMIT) {
        // o^T = fo o (S^T q^T) + x^T P^T.  Tile o[mt][nt] holds value columns
        // c0 + 16 nt + 4(lane/16) + j of token 16 mt + lane%16, so fo is one
        // factor per lane, x fragments are the A operands and the P fragments
        // (rows = tokens) the B operands.
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
          const float fo = C.fo[16 * mt + ln];
#pragma unroll
          for (int nt = 0; nt < NN; nt++) o[mt][nt] *= fo;
        }
#pragma unroll
        for (int s = 0; s < NSB; s++) {
          Fr xs[NN];
#pragma unroll
          for (int nt = 0; nt < NN; nt++) xs[nt] = acc_as_b<O>(x, s, nt);
#pragma unroll
          for (int mt = 2 * s; mt < 4; mt++) {
            const Fr pf = *reinterpret_cast<const Fr*>(C.p + p_frag(mt, s) * 1024 + lane * 16);
#pragma unroll
            for (int nt = 0; nt < NN; nt++) M::mma(o[mt][nt], xs[nt], pf);
          }
        }
      }
      // S <- eC S + k^T (fd o x)
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const floatx4 fd = *reinterpret_cast<const floatx4*>(Fd + 16 * mt + 4 * g4);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) x[mt][nt] *= fd;
      }
      Fr xv[NSB][NN];
#pragma unroll
      for (int s = 0; s < NSB; s++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++) xv[s][nt] = acc_as_b<O>(x, s, nt);
#pragma unroll
      for (int mt = 0; mt < DKT; mt++) {
        floatx4 acc[NN];
#pragma unroll
        for (int nt = 0; nt < NN; nt++) acc[nt] = S[mt][nt] * eC;
#pragma unroll
        for (int s = 0; s < NSB; s++) {
          // A = k^T: the dk rows of tile mt (permuted), tokens s KS.. down the
          // stored rows
          const int cdk = 32 * (mt >> 1) + 4 * (mt & 1);
          const bf16x4 lo = lds_rows4_tr(C.k, SM::LDK, s * KS, cdk, lane, 8);
          const bf16x4 hi = lds_rows4_tr(C.k, SM::LDK, s * KS + 16, cdk, lane, 8);
          const Fr kf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int nt = 0; nt < NN; nt++) M::mma(acc[nt], kf, xv[s][nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NN; nt++) S[mt][nt] = acc[nt];
      }
      if (mcol && log_norm < kNegligibleLog) {
        m_zero = true;
#pragma unroll
        for (int mt = 0; mt < DKT; mt++)
#pragma unroll
          for (int nt = 0; nt < NN; nt++) S[mt][nt] = zero4();
      }
      if constexpr (OUT && EMIT) {
        // o, after the state update's products (which hide the latency of
        // the last o products): four consecutive value columns of one token
        // per lane, one 8-byte (bf16) store per tile, straight to HBM
        // (a buffer resource over the chunk's rows of this head: the
        // lane's byte offset is fixed, rows past the sequence end fall
        // outside the range and their stores are dropped)
        typedef E E4 __attribute__((ext_vector_type(4)));
        static_assert(sizeof(E4) == 8, "8-byte o stores");
        const int64_t tc = tb + (int64_t)it * BT;
        const int64_t rows = te - tc < BT ? te - tc : BT;
        const __amdgpu_buffer_rsrc_t ro =
            buffer_rsrc((E*)a.o + (tc * o_ld + (int64_t)h * DV),
                        (uint32_t)(((rows - 1) * o_ld + DV) * (int64_t)sizeof(E)));
        const uint32_t ooff = (uint32_t)((ln * o_ld + c0 + 4 * g4) * (int64_t)sizeof(E));
#pragma unroll
        for (int mt = 0; mt < 4; mt++) {
#pragma unroll
          for (int nt = 0; nt < NN; nt++) {
            E4 v4;
#pragma unroll
            for (int j = 0; j < 4; j++) v4[j] = from_f<E>(o[mt][nt][j]);
            buffer_store8(v4, ro, ooff, (uint32_t)((16 * mt * o_ld + 16 * nt) * (int64_t)sizeof(E)));
          }
        }
      }
  };
  lds_barrier();  // the first chunk is published
  for (int it = -nwarm; it < 0; it++) {
    step(std::false_type{}, buf[it & 1], it);
    lds_barrier();
  }
  for (int it = 0; it < nchunks; it++) {
    if (!(mcol && m_zero)) step(std::true_type{}, buf[it & 1], it);
    lds_barrier();
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
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int row = dk_of_row(mt, 4 * g4 + j), col = c0 + 16 * nt + ln;
          dst[row * ld + col] = S[mt][nt][j];
        }
  }
}

template <typename E, int DK, int DV, int MODE>
__global__ __launch_bounds__((WsCfg<E, DK, DV, MODE>::NT)) void chunk_ws_kernel(LoopArgs a) {
  typedef typename WsCfg<E, DK, DV, MODE>::SM SM;
  __shared__ SM buf[2];
  __shared__ unsigned p_count;  // loader waves' stored chunks, a running count (P hand-off)
  if (is_out(MODE)) {
    if (threadIdx.x == 0) p_count = 0u;
    __syncthreads();
  }
  // Workgroup order: the value heads of one q/k head and segment take ids 8
  // apart, so they run together on one XCD (ids go round-robin over the 8
  // XCDs) and share q and k through its L2; with a span of 8 segments, XCD x
  // runs segment x of every head.
  const int GR = a.Hv / a.Hk;
  const int id = blockIdx.x;
  const int grp = (id / (8 * GR)) * 8 + (id & 7), member = (id >> 3) % GR;
  const int seg = grp % a.seg_span, h = (grp / a.seg_span) * GR + member;
  if (grp >= a.seg_span * a.Hk || seg >= a.counts[0]) return;
  const int4 ent = a.seg_table[seg];
  if (MODE == kSummary && (ent.w & kLast) && !a.summary_all) return;
  // a replaying sequence needs no summaries
  if (MODE == kSummary && a.seq_warm && a.seq_warm[(int64_t)ent.x * a.Hv + h]) return;
  ws_body<E, DK, DV, MODE>(a, buf, &p_count, seg, h, ent);
}

// Scan over segment summaries (fp32): per (sequence, head, 16 columns),
// h <- M h + E over the segments of the sequence, with fp32 MFMA products
// (wave w owns rows 32 w .. 32 w + 31 of h; M's rows are the A operands,
// read straight from the summaries, h the B operand from LDS).  Forward:
// from h0 over segments 0 .. nseg - 2, giving the initial states of 1 ..
// nseg - 1.  REV (the backward's dS): from dht over segments nseg - 1 .. 1,
// giving the state gradient leaving segments nseg - 2 .. 0.
template <int DK, int DV, bool REV = false>
__global__ __launch_bounds__(DK * 2) void seg_scan_kernel(const float* __restrict__ seg_state,
                                                          float* __restrict__ seg_init,
                                                          const float* __restrict__ h0,
                                                          const int32_t* __restrict__ seq_off,
                                                          const int32_t* __restrict__ seq_nseg, int Hv,
                                                          const int32_t* __restrict__ seq_warm = nullptr) {
  typedef Mfma<float> M;
  constexpr int LDX = DK + DV;
  constexpr int NKT = DK / 16;
  static_assert(DK % 32 == 0, "two row tiles per wave");
  const int n = blockIdx.x, h = blockIdx.y, cb = blockIdx.z * 16;
  const int nseg = seq_nseg[n];
  if (nseg <= 1) return;
  if (seq_warm && seq_warm[(int64_t)n * Hv + h]) return;  // replayed, no summaries
  const int off = seq_off[n];
  __shared__ float hs[DK][16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g4 = lane >> 4, ln = lane & 15;
  for (int i = t; i < DK * 16; i += DK * 2) {
    const int r = i >> 4, col = i & 15;
    hs[r][col] = h0 ? h0[(((int64_t)n * Hv + h) * DK + r) * DV + cb + col] : 0.f;
  }
  __syncthreads();
  for (int i = 0; i + 1 < nseg; i++) {
    const int p = REV ? nseg - 1 - i : i;  // the summary applied
    const int q = REV ? p - 1 : p + 1;     // the segment whose state it gives
    const float* X = seg_state + ((int64_t)(off + p) * Hv + h) * DK * LDX;
    floatx4 acc[2];
    floatx4 af[2][NKT];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int mt = 2 * w + i;
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = X[(16 * mt + 4 * g4 + j) * LDX + DK + cb + ln];
#pragma unroll
      for (int kt = 0; kt < NKT; kt++) af[i][kt] = M::load(X, LDX, 16 * mt, 16 * kt, lane);
    }
#pragma unroll
    for (int kt = 0; kt < NKT; kt++) {
      const floatx4 bf = M::load_col(&hs[0][0], 16, 0, 16 * kt, lane);
#pragma unroll
      for (int i = 0; i < 2; i++) M::mma(acc[i], af[i][kt], bf);
    }
    __syncthreads();  // every wave has read h
    float* dst = seg_init + ((int64_t)(off + q) * Hv + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int r = 16 * (2 * w + i) + 4 * g4 + j;
        hs[r][ln] = acc[i][j];
        dst[r * DV + cb + ln] = acc[i][j];
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

// bfloat16 runs the prepared-chunk state pass (its two buffers fit in LDS);
// float32 the single-buffer chunk loop.
template <typename E, int DK, int DV, int MODE>
constexpr bool uses_prep() {
  if constexpr (std::is_same<E, bf16>::value)
    return WsCfg<E, DK, DV, MODE>::FITS && WsCfg<E, DK, DV, kSummary>::FITS;
  else
    return false;
}

// One pass of the chunk loop over every segment.
template <typename E, int DK, int DV, int MODE>
void launch_loop(const LoopArgs& a, const Plan& pl, hipStream_t stream) {
  const dim3 grid((unsigned)pl.seg_cap, a.Hv);
  if constexpr (uses_prep<E, DK, DV, MODE>()) {
    const int64_t unit = 8 * (int64_t)(a.Hv / a.Hk);
    const int64_t n = ((int64_t)a.seg_span * a.Hv + unit - 1) / unit * unit;
    hipLaunchKernelGGL((chunk_ws_kernel<E, DK, DV, MODE>), dim3((unsigned)n),
                       dim3(WsCfg<E, DK, DV, MODE>::NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((chunk_loop_kernel<E, DK, DV, MODE>), grid, dim3(LoopCfg<E, DK, DV, MODE>::NT),
                       0, stream, a);
  }
}

// Plan, summaries + scan when segments split a sequence, then the final pass
// in `FINAL` mode (kOut, kOutSave or kStates).  `a` carries the caller's tensors;
// rec_buf, if not null, takes the prepared records instead of the workspace.
template <typename E, int DK, int DV, int FINAL>
int run_pipeline(LoopArgs a, const int32_t* cu, int N, int64_t T, const Plan& pl, char* ws,
                 bool with_chunks, hipStream_t stream, char* rec_buf = nullptr) {
  constexpr bool PREP = uses_prep<E, DK, DV, FINAL>();
  PlanPtrs pp = pl.ptrs(ws, with_chunks || PREP);
  a.seg_cap = (int)pl.seg_cap;
  a.seg_table = pp.table;
  a.counts = pp.counts;
  a.seg_chunk0 = pp.seg_chunk0;
  a.seg_state = pl.split ? reinterpret_cast<float*>(ws + pl.off_state) : nullptr;
  a.seg_init = pl.split ? reinterpret_cast<float*>(ws + pl.off_init) : nullptr;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, (int)pl.seg_first, (int)pl.seg_len,
                     (int)pl.seg_cap, (int)pl.chunk_cap, pp);
  if (int rc = gdn::check_launch("chunk plan")) return rc;
  if constexpr (PREP) {
    char* rec = rec_buf ? rec_buf : ws + pl.off_rec;
    a.rec = rec;
    PrepArgs pa{a.k, a.ld_qk, prep_gates(a), a.Hk, a.Hv, a.use_l2norm, pp.chunk_tab,
                pp.counts, rec};
    if (int rc = launch_prep<DK>(pa, pl.chunk_cap, stream)) return rc;
    if (pl.split) {
      // per (sequence, head): replay instead of summaries where the records'
      // bounds allow it
      int32_t* warm = reinterpret_cast<int32_t*>(ws + pl.off_warm);
      int32_t* seq_warm = reinterpret_cast<int32_t*>(ws + pl.off_seq_warm);
      hipLaunchKernelGGL(warm_kernel, dim3(N, a.Hv), dim3(256), 0, stream, rec, a.Hv, pp.counts,
                         pp.seg_chunk0, pp.seq_off, pp.seq_nseg, pp.seq_chunk_off, (int)pl.seg_cap,
                         warm, seq_warm);
      if (int rc = gdn::check_launch("chunk replay table")) return rc;
      a.warm = warm;
      a.seq_warm = seq_warm;
    }
  }
  a.seg_span = (int)pl.seg_span;
  if (pl.split) {
    launch_loop<E, DK, DV, kSummary>(a, pl, stream);
    if (int rc = gdn::check_launch("chunk summary")) return rc;
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV>), dim3(N, a.Hv, DV / 16), dim3(DK * 2), 0, stream,
                       a.seg_state, a.seg_init, a.h0, pp.seq_off, pp.seq_nseg, a.Hv, a.seq_warm);
    if (int rc = gdn::check_launch("chunk scan")) return rc;
  }
  launch_loop<E, DK, DV, FINAL>(a, pl, stream);
  return gdn::check_launch("chunk loop");
}

// Composition of a sequence's segment summaries into the summary of the whole
// sequence (hyper-parallel _compute_gdn_state_summary_from_prepared, folded
// over segments instead of chunks): per (sequence, head, 16 columns of
// [M | E]), X <- M_p X + [0 | E_p] over its segments from X = [I | 0]; an
// empty sequence gives [I | 0].  fp32 MFMA tiles as in seg_scan_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(DK * 2) void seg_compose_kernel(const float* __restrict__ seg_state,
                                                             const int32_t* __restrict__ seq_off,
                                                             const int32_t* __restrict__ seq_nseg,
                                                             int Hv, float* __restrict__ Mout,
                                                             float* __restrict__ Eout) {
  typedef Mfma<float> M;
  constexpr int LDX = DK + DV;
  constexpr int NKT = DK / 16;
  static_assert(DK % 32 == 0, "two row tiles per wave");
  const int n = blockIdx.x, h = blockIdx.y, cb = blockIdx.z * 16;
  const bool ecol = cb >= DK;  // the block holds columns of E
  float* dst = ecol ? Eout : Mout;
  if (!dst) return;
  const int nseg = seq_nseg[n], off = seq_off[n];
  __shared__ float hs[DK][16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g4 = lane >> 4, ln = lane & 15;
  for (int i = t; i < DK * 16; i += DK * 2) {
    const int r = i >> 4, col = i & 15;
    hs[r][col] = (!ecol && r == cb + col) ? 1.f : 0.f;
  }
  __syncthreads();
  for (int p = 0; p < nseg; p++) {
    const float* X = seg_state + ((int64_t)(off + p) * Hv + h) * DK * LDX;
    floatx4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int mt = 2 * w + i;
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = ecol ? X[(16 * mt + 4 * g4 + j) * LDX + cb + ln] : 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; kt++)
        M::mma(acc[i], M::load(X, LDX, 16 * mt, 16 * kt, lane), M::load_col(&hs[0][0], 16, 0, 16 * kt, lane));
    }
    __syncthreads();  // every wave has read the running summary
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) hs[16 * (2 * w + i) + 4 * g4 + j][ln] = acc[i][j];
    __syncthreads();
  }
  const int ld = ecol ? DV : DK, c0 = ecol ? cb - DK : cb;
  float* out = dst + ((int64_t)n * Hv + h) * DK * ld;
  for (int i = t; i < DK * 16; i += DK * 2) {
    const int r = i >> 4, col = i & 15;
    out[r * ld + c0 + col] = hs[r][col];
  }
}

// Prefix merge of affine summaries (hyper-parallel
// _merge_gdn_prefix_state_summaries_torch, and _apply_gdn_state_summary for
// one summary): per (state slot, 16 columns), h <- M_r h + E_r for
// r = 0 .. R-1 from h_in (zero if null).  M [R][S][DK][DK], E [R][S][DK][DV].
template <int DK, int DV>
__global__ __launch_bounds__(DK * 2) void merge_summaries_kernel(const float* __restrict__ Ms,
                                                                 const float* __restrict__ Es,
                                                                 int R, int S,
                                                                 const float* __restrict__ h_in,
                                                                 float* __restrict__ h_out) {
  typedef Mfma<float> M;
  constexpr int NKT = DK / 16;
  static_assert(DK % 32 == 0, "two row tiles per wave");
  const int sl = blockIdx.x, cb = blockIdx.y * 16;
  __shared__ float hs[DK][16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g4 = lane >> 4, ln = lane & 15;
  for (int i = t; i < DK * 16; i += DK * 2) {
    const int r = i >> 4, col = i & 15;
    hs[r][col] = h_in ? h_in[((int64_t)sl * DK + r) * DV + cb + col] : 0.f;
  }
  __syncthreads();
  for (int p = 0; p < R; p++) {
    const float* Mp = Ms + ((int64_t)p * S + sl) * DK * DK;
    const float* Ep = Es + ((int64_t)p * S + sl) * DK * DV;
    floatx4 acc[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int mt = 2 * w + i;
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = Ep[(16 * mt + 4 * g4 + j) * DV + cb + ln];
#pragma unroll
      for (int kt = 0; kt < NKT; kt++)
        M::mma(acc[i], M::load(Mp, DK, 16 * mt, 16 * kt, lane), M::load_col(&hs[0][0], 16, 0, 16 * kt, lane));
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) hs[16 * (2 * w + i) + 4 * g4 + j][ln] = acc[i][j];
    __syncthreads();
  }
  for (int i = t; i < DK * 16; i += DK * 2) {
    const int r = i >> 4, col = i & 15;
    h_out[((int64_t)sl * DK + r) * DV + cb + col] = hs[r][col];
  }
}

// A shard's affine summary per local sequence: plan, prep (bf16), the
// summary pass over every segment (last ones included), then the
// composition over each sequence's segments into M and E.
template <typename E, int DK, int DV>
int run_summary(LoopArgs a, const int32_t* cu, int N, int64_t T, const Plan& pl, char* ws,
                float* Mout, float* Eout, hipStream_t stream) {
  constexpr bool PREP = uses_prep<E, DK, DV, kSummary>();
  PlanPtrs pp = pl.ptrs(ws, PREP);
  a.seg_cap = (int)pl.seg_cap;
  a.seg_table = pp.table;
  a.counts = pp.counts;
  a.seg_chunk0 = pp.seg_chunk0;
  a.seg_state = reinterpret_cast<float*>(ws + pl.off_state);
  a.seg_init = nullptr;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, (int)pl.seg_first, (int)pl.seg_len,
                     (int)pl.seg_cap, (int)pl.chunk_cap, pp);
  if (int rc = gdn::check_launch("chunk plan")) return rc;
  if constexpr (PREP) {
    char* rec = ws + pl.off_rec;
    a.rec = rec;
    PrepArgs pa{a.k, a.ld_qk, prep_gates(a), a.Hk, a.Hv, a.use_l2norm, pp.chunk_tab, pp.counts, rec};
    if (int rc = launch_prep<DK>(pa, pl.chunk_cap, stream)) return rc;
  }
  a.seg_span = (int)pl.seg_span;
  a.summary_all = 1;
  launch_loop<E, DK, DV, kSummary>(a, pl, stream);
  if (int rc = gdn::check_launch("chunk summary")) return rc;
  hipLaunchKernelGGL((seg_compose_kernel<DK, DV>), dim3(N, a.Hv, (DK + DV) / 16), dim3(DK * 2), 0,
                     stream, a.seg_state, pp.seq_off, pp.seq_nseg, a.Hv, Mout, Eout);
  return gdn::check_launch("chunk summary compose");
}

}  // namespace
}  // namespace gdn_chunk
