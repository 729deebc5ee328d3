// chunk_bwd.hip -- gdn_chunk_bwd: reverse mode of the chunked gated delta
// rule (gdn_chunk_fwd), l2norm and GQA head sharing included.
//
// Gradient contract: hyper-parallel "linear_attention_context_parallel.py",
// _RecvInitialStateP2PFunction / _SendFinalStateP2PFunction -- the gradient
// of the final state (dht) comes in, the gradient of the initial state (dh0)
// goes out.  The math is the adjoint of the chunk algorithm of
// _prepare_gdn_chunks_for_summary / _run_prepared_gdn_chunks.  Per chunk,
// with S the state entering it, S' the state leaving it, gamma = e^G,
// D = e^{G_C - G}, Vn = u - w S (v_new) and dS' = dL/dS':
//   dVn  = P^T dO + D o (K dS')
//   dS   = gamma_C dS' + Q^T (gamma o dO) - W^T dVn          (carried back)
//   Y    = T^T dVn                   (gradient of u = T beta v, through T)
//   dv   = beta o Y
//   dQ   = gamma o (dO S^T) + dA K,        dA = (dO Vn^T) o Gamma, i >= j
//   dK   = dA^T Q + D o (Vn dS'^T) - beta gamma o (Y S^T) + (M1 + M1^T) K
//   M1   = diag(beta) (dL o Gamma) with dL = -Y Vn^T, strict lower
// The last two use the identities  T^T dW = -Y S^T  (dW = -dVn S^T) and
//   dL = -(Y u^T + T^T dW w^T) = -Y (u - w S)^T = -Y Vn^T,
// so the w-path needs no extra [64, dk] intermediates.  dbeta and dG are row
// sums of the same products; dg is the reverse in-chunk cumsum of dG.
//
// Kernels:
//   1. the forward pipeline in "states" mode stores the state entering every
//      chunk (fp32), with the segment summaries for parallelism;
//   2. dstate: per (sequence, head), chunks in reverse, carries dS and stores
//      dS' of every chunk (fp32); writes dh0;
//   3. grad: per (chunk, head), all local gradients from S and dS' (fully
//      parallel); dq-hat, dk-hat per value head go to an fp32 buffer;
//   4. finalize: per (token, q/k head), sum over the value heads sharing it and
//      back through l2norm and scale into the dq, dk views.
#include <hip/hip_runtime.h>

#include "chunk_loop.h"
#include "gdn_internal.h"

using namespace gdn_chunk;


namespace {

struct BwdArgs {
  const void* q;
  const void* k;
  int64_t ld_qk;
  const void* v;
  int64_t ld_v;
  const float* g;
  const float* beta;
  int Hk, Hv;
  float scale;
  int use_l2norm;
  const void* d_o;
  const float* dht;
  void* dq;
  void* dk;
  int64_t ld_dqk;
  void* dv;
  int64_t ld_dv;
  float* dg;
  float* dbeta;
  float* dh0;
  const int32_t* cu;
  int64_t T;
  const int32_t* counts;
  const int4* chunk_tab;
  const int32_t* seq_chunk_off;
  // the state entering / the state gradient leaving every chunk,
  // [chunk_cap][Hv][DK][DV] in the activation type (they feed MFMAs of that
  // type only)
  const void* states;
  void* dstates;
  float* dqk;           // [T][Hv][2][DK]
  // segments of the sequences (the forward plan's), for the dS pass
  const int4* seg_table;
  const int32_t* seg_chunk0;
  float* seg_sum;       // [seg_cap][Hv][DK][DK+DV] reverse summaries [M | E]
  float* seg_in;        // [seg_cap][Hv][DK][DV] dS leaving each non-last segment
  // the forward prep's records [chunk_cap][Hv] (bfloat16 only, else null):
  // T = (I + diag(beta) L)^-1 diag(beta) as MFMA A fragments
  const char* rec;
  // replay of the dS recurrence (warm_rev_kernel): per (segment, head) the
  // chunks after the segment its final pass runs first, from zero (|
  // kWarmFromStart: from the sequence end, with dht); per (sequence, head) 1
  // when every segment but the last replays (then no dS summaries or scan).
  // Null: summaries and scan as usual.
  const int32_t* rev_warm;
  const int32_t* seq_rev_warm;
};

// The replay table of the dS recurrence: the mirror of warm_kernel.  The
// chunk's adjoint map dS' -> dS is the transpose of its forward transition,
// with the same norm, so the records' bounds lb serve here too, summed
// forwards from the end of every segment but a sequence's last.
__global__ __launch_bounds__(256) void warm_rev_kernel(const char* __restrict__ rec, int Hv,
                                                       const int32_t* __restrict__ counts,
                                                       const int4* __restrict__ seg_table,
                                                       const int32_t* __restrict__ seg_chunk0,
                                                       const int32_t* __restrict__ seq_off,
                                                       const int32_t* __restrict__ seq_nseg,
                                                       int seg_cap, int32_t* __restrict__ warm,
                                                       int32_t* __restrict__ seq_warm) {
  const int n = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int off = seq_off[n], nseg = seq_nseg[n];
  const int nchunks = counts[1];
  int cold = 0;
  if (nseg > 1 && off + nseg - 1 < seg_cap) {
    const int4 last = seg_table[off + nseg - 1];
    const int clast = seg_chunk0[off + nseg - 1] + (last.z - last.y + BT - 1) / BT - 1;
    for (int p = t; p + 1 < nseg; p += 256) {
      const int s = off + p;
      const int4 e = seg_table[s];
      const int ce = seg_chunk0[s] + (e.z - e.y + BT - 1) / BT;  // first chunk after it
      int val = -1;
      float sum = 0.f;
      for (int w = 0; w < kWarmMax; w++) {
        const int c = ce + w;
        if (c > clast) {  // the sequence end: replay all of it, from dht
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
  } else if (nseg > 1) {
    cold = 1;
  }
  cold = __syncthreads_or(cold);
  if (t == 0) seq_warm[(int64_t)n * Hv + h] = cold ? 0 : 1;
}

// w = T diag(beta e^G) kh of one chunk from the prep's record: with the
// record's T_r = (I + diag(beta) L)^-1 diag(beta) that is T_r diag(e^G) kh, a
// product of the stored fragments (no gram, inversion or solve again).  Each
// wave forms the tiles of one row block (mt = wave % 4), whose T fragments it
// read from the record into tf.
template <int DK, int NW, class SM>
GDN_DEV void compute_w_rec(SM& sm, int wave, int lane, const bf16x8 (&tf)[2]) {
  typedef Mfma<bf16> M;
  static_assert(NW % 4 == 0, "one row block a wave");
  constexpr int NTILE = 4 * (DK / 16);
  const int mt = wave % 4;
  for (int tt = wave; tt < NTILE; tt += NW) {
    const int nt = tt / 4;
    floatx4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 2; s++)
      if (2 * s <= mt)  // the fragments right of the diagonal are zero
        M::mma(acc, tf[s], M::load_col_scaled(sm.k, SM::LDK, 16 * nt, s * M::KSTEP, sm.eg, lane));
    const int rb = 16 * mt + 4 * (lane >> 4), c = 16 * nt + (lane & 15);
#pragma unroll
    for (int jj = 0; jj < 4; jj++) sm.w[(rb + jj) * SM::LDK + c] = from_f<bf16>(acc[jj]);
  }
}

#ifndef GDN_GRAD_CW
#define GDN_GRAD_CW 16
#endif
template <typename E, int DK, int DV>
struct BwdCfg {
  typedef E O;
  // value columns a wave: 16 (eight waves, two a SIMD, at dv = 128) while
  // that leaves at least four waves, else 32
  static constexpr int CW = DV / GDN_GRAD_CW >= 4 ? GDN_GRAD_CW : 32;
  static constexpr int NW = DV / CW;
  static constexpr int NT = NW * 64;
  typedef Smem<O, DK, DV, true> SM;
  typedef Prefetch<E, DK, DV, NT, true> PF;
};

// dS pass: 32 state columns a wave; the summary mode carries the extended
// state [M | E] (DK + DV columns) in one workgroup, so the chunk's shared
// work (gram, T, w) is formed once for both.
#ifndef GDN_DS_CW_SUM
#define GDN_DS_CW_SUM 32
#endif
#ifndef GDN_DS_CW_FIN
#define GDN_DS_CW_FIN 16
#endif
template <typename E, int DK, int DV, bool SUM>
struct DsCfg {
  typedef E O;
  // state columns a wave: the final pass's waves hold 16 (eight waves, two a
  // SIMD, at dv = 128), the summary's 32 (its 256 columns in eight waves)
  static constexpr int COLS = SUM ? DK + DV : DV;
  static constexpr int CW_REQ = SUM ? GDN_DS_CW_SUM : GDN_DS_CW_FIN;
  static constexpr int CW = COLS / CW_REQ >= 4 ? CW_REQ : 32;  // at least four waves, else 32
  static constexpr int NW = COLS / CW;
  static constexpr int NT = NW * 64;
  typedef Smem<O, DK, DV, true> SM;
  typedef Prefetch<E, DK, DV, NT, true> PF;
};

// ---------------------------------------------------------------------------
// 2. dS pass: reverse over the chunks of one segment
// ---------------------------------------------------------------------------
// Per chunk, dS = (gamma_C I - W^T diag(D) K) dS' + Q^T (gamma o dO) - W^T P^T dO
// is affine in dS', so the forward's segments serve here too: the summary
// mode (SUM) runs a segment on the extended state [I | 0] (no dO for the
// identity columns) from its end back to its start, giving dS_in = M dS_out +
// E for every segment but a sequence's first; a reverse scan folds them from
// dht; the final mode runs every segment from its own dS_out, stores dS' of
// each chunk and writes dh0 in the first segment.
template <typename E, int DK, int DV, bool SUM>
__global__ __launch_bounds__((DsCfg<E, DK, DV, SUM>::NT)) void dstate_kernel(BwdArgs a) {
  typedef DsCfg<E, DK, DV, SUM> CF;
  typedef typename CF::O O;
  typedef Mfma<O> M;
  typedef typename CF::SM SM;
  constexpr int NW = CF::NW, NT = CF::NT, KS = M::KSTEP, CW = CF::CW, NN = CW / 16;
  constexpr int NSK = DK / KS, NSB = BT / KS, DKT = DK / 16;
  __shared__ SM sm;  // sm.v holds the chunk of dO

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= a.counts[0]) return;
  const int4 ent = a.seg_table[seg];
  if (SUM && (ent.w & kFirst)) return;
  const int n = ent.x;
  const bool replay = a.seq_rev_warm && a.seq_rev_warm[(int64_t)n * a.Hv + blockIdx.y];
  if (SUM && replay) return;  // no summaries needed
  const int Hv = a.Hv, qa = h / (Hv / a.Hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c0 = wave * CW;                 // first (extended) state column
  const bool mcol = SUM && c0 < DK;         // columns of M: no dO
  const int vc0 = SUM ? c0 - DK : c0;       // value column of the first column
  const int64_t s0 = ent.y, e0 = ent.z;
  const int nch = (int)((e0 - s0 + BT - 1) / BT);
  const int chunk0 = a.seg_chunk0[seg];
  // final pass of a replaying sequence: the chunks after the segment run
  // first (no dS' stores), from zero or, reaching the sequence end, from dht
  int nwarm = 0;
  bool warm_dht = false;
  if (!SUM && replay && !(ent.w & kLast)) {
    const int v = a.rev_warm[(int64_t)seg * Hv + h];
    nwarm = v & ~kWarmFromStart;
    warm_dht = (v & kWarmFromStart) != 0;
  }
  // rows past the sequence end are zero (replayed chunks lie beyond e0)
  const int64_t te = nwarm > 0 ? (a.cu[n + 1] < a.T ? (int64_t)a.cu[n + 1] : a.T) : e0;

  zero_upper<O, true, NT>(sm, tid);
  floatx4 dS[DKT][NN];
  {
    const float* src = nullptr;
    if (!SUM) {
      const float* dhtn = a.dht ? a.dht + ((int64_t)n * Hv + h) * DK * DV : nullptr;
      if (nwarm > 0) src = warm_dht ? dhtn : nullptr;
      else if (!(ent.w & kLast)) src = a.seg_in + ((int64_t)seg * Hv + h) * DK * DV;
      else src = dhtn;
    }
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int row = 16 * mt + 4 * (lane >> 4) + j, col = c0 + 16 * nt + (lane & 15);
          float v = 0.f;
          if (mcol) v = row == col ? 1.f : 0.f;
          else if (src) v = src[row * DV + col];
          dS[mt][nt][j] = v;
        }
  }
  const E* qp = (const E*)a.q + (int64_t)qa * DK;
  const E* kp = (const E*)a.k + (int64_t)qa * DK;
  const E* dop = (const E*)a.d_o + (int64_t)h * DV;
  const float* gp = a.g + h;
  const float* bp = a.beta + h;
  typename CF::PF pf;
  const int ctop = nch - 1 + nwarm;  // chunks ctop .. nch are replayed
  if (nch > 0) pf.load(qp, kp, a.ld_qk, dop, (int64_t)Hv * DV, gp, bp, Hv, s0 + (int64_t)ctop * BT, te, tid);

  for (int c = ctop; c >= 0; c--) {
    const int64_t tc = s0 + (int64_t)c * BT;
    __syncthreads();
    stage<E, O, DK, DV, NT, true>(sm, pf, a.scale, a.use_l2norm, tid);
    if (c > 0) pf.load(qp, kp, a.ld_qk, dop, (int64_t)Hv * DV, gp, bp, Hv, tc - BT, te, tid);
    if (!SUM && c < nch) {  // dS' of this chunk for the gradient kernel
      E* dst = (E*)a.dstates + ((int64_t)(chunk0 + c) * Hv + h) * DK * DV;
#pragma unroll
      for (int mt = 0; mt < DKT; mt++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            dst[(16 * mt + 4 * (lane >> 4) + j) * DV + c0 + 16 * nt + (lane & 15)] =
                from_f<E>(dS[mt][nt][j]);
    }
    __syncthreads();
    if constexpr (std::is_same<E, bf16>::value && NW % 4 == 0) {
      // T from the forward prep's record (this wave's row block), P tiles on
      // every wave
      bf16x8 tf[2];
      {
        const int mt = wave % 4;
        const char* R = a.rec + ((int64_t)(chunk0 + c) * Hv + h) * kRecBytes + kRecT + lane * 16;
#pragma unroll
        for (int s2 = 0; s2 < 2; s2++)
          tf[s2] = 2 * s2 <= mt ? *reinterpret_cast<const bf16x8*>(R + p_frag(mt, s2) * 1024) : bf16x8{};
      }
      for (int t = wave; t < 10; t += NW) {
        int ti, tj;
        lower_tile_ij(t, ti, tj);
        gram_tile<O, DK>(sm, true, ti, tj, lane);
      }
      compute_w_rec<DK, NW>(sm, wave, lane, tf);
    } else {
      gram_kk<O, DK, NW>(sm, wave, lane);
      __syncthreads();
      solve<O, DK, NW, true>(sm, wave, lane);
      compute_w<O, DK, NW>(sm, wave, lane);
    }
    __syncthreads();

    const float GC = sm.G[BT - 1];
    // dVn = P^T dO + D o (K dS')
    typename M::frag sb[NSK][NN];
#pragma unroll
    for (int s = 0; s < NSK; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) sb[s][nt] = acc_as_b<O>(dS, s, nt);
    floatx4 dvn[4][NN];
    // this wave's dO columns (the identity columns see no dO: their operand
    // is zero -- a select, not a branch, keeps both modes' registers alike)
    typename M::frag dof[NSB][NN];
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        const typename M::frag vv = M::load_col(sm.v, SM::LDV, (vc0 < 0 ? 0 : vc0) + 16 * nt, s * KS, lane);
        dof[s][nt] = mcol ? typename M::frag{} : vv;
      }
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      floatx4 kk[NN], pp[NN];
#pragma unroll
      for (int nt = 0; nt < NN; nt++) kk[nt] = pp[nt] = zero4();
#pragma unroll
      for (int s = 0; s < NSK; s++) {
        const typename M::frag kf = M::load(sm.k, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(kk[nt], kf, sb[s][nt]);
      }
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        const typename M::frag pt = M::load_col(sm.p, SM::LDT, 16 * mt, s * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(pp[nt], pt, dof[s][nt]);
      }
      const int rb = 16 * mt + 4 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float d = __expf(GC - sm.G[rb + j]);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) pp[nt][j] += d * kk[nt][j];
      }
#pragma unroll
      for (int nt = 0; nt < NN; nt++) dvn[mt][nt] = -pp[nt];  // negated: the W^T term enters with a minus
    }
    // dS <- gamma_C dS' + Q^T (gamma o dO) - W^T dVn
    const float eC = __expf(GC);
    typename M::frag db[NSB][NN], gb[NSB][NN];
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        db[s][nt] = acc_as_b<O>(dvn, s, nt);
        const typename M::frag gv =
            M::load_col_scaled(sm.v, SM::LDV, (vc0 < 0 ? 0 : vc0) + 16 * nt, s * KS, sm.eg, lane);
        gb[s][nt] = mcol ? typename M::frag{} : gv;
      }
#pragma unroll
    for (int mt = 0; mt < DKT; mt++) {
      floatx4 acc[NN];
#pragma unroll
      for (int nt = 0; nt < NN; nt++) acc[nt] = dS[mt][nt] * eC;
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        const typename M::frag qt = M::load_col(sm.q, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(acc[nt], qt, gb[s][nt]);
        const typename M::frag wt = M::load_col(sm.w, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(acc[nt], wt, db[s][nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NN; nt++) dS[mt][nt] = acc[nt];
    }
  }
  // the summary [M | E] of the segment, or dh0 from a sequence's first segment
  float* dst = nullptr;
  int ld = DV;
  if (SUM) {
    dst = a.seg_sum + ((int64_t)seg * Hv + h) * DK * (DK + DV);
    ld = DK + DV;
  } else if ((ent.w & kFirst) && a.dh0) {
    dst = a.dh0 + ((int64_t)n * Hv + h) * DK * DV;
  }
  if (dst) {
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          dst[(16 * mt + 4 * (lane >> 4) + j) * ld + c0 + 16 * nt + (lane & 15)] = dS[mt][nt][j];
  }
}

// ---------------------------------------------------------------------------
// 2b. dS final pass with the forward state pass's loader / consumer split
// ---------------------------------------------------------------------------
// Per chunk, with dS' the state gradient leaving it (carried back from the
// chunk after), the adjoint of the state pass's three steps
//   x = T (v - fk o (k S)),  o = fo o (q S) + P x,  S' = eC S + k^T (fd o x)
// is
//   dx = P^T dO + fd o (k dS'),   dy = T^T dx,
//   dS = eC dS' + q^T (fo o dO) - k^T (fk o dy).
// Four loader waves stage q, k, dO and the record of the chunk before (the
// chunks run in reverse) and make P^T and T^T as A fragments; dv / 32 consumer
// waves carry 32 columns of dS each in MFMA accumulators (dk rows permuted as
// in the forward), store dS' of every chunk for the gradient kernel and write
// dh0 at a sequence's first segment.  Replay and the initial dS as in
// dstate_kernel's final mode.

// Halves of P^T being made by the loaders: (row block mt of P^T = token block
// of k, token block jq of q), the two that lie below the diagonal (all zero)
// last.
constexpr int kPtHalves = 12;
__host__ __device__ constexpr int pt_half_mt(int u) {
  return u < 4 ? 0 : u < 7 ? 1 : u < 9 ? 2 : u == 9 ? 3 : u == 10 ? 1 : 3;
}
__host__ __device__ constexpr int pt_half_jq(int u) {
  return u < 4 ? u : u < 7 ? u - 3 : u < 9 ? u - 5 : u == 9 ? 3 : u == 10 ? 0 : 2;
}

// Half (mt, jq): the tile q_jq k_mt^T (rows = tokens tok of q, columns =
// tokens tok' of k) holds in lane l the elements P[tok = 16 jq + 4(l/16) + e]
// [tok' = 16 mt + l%16], exactly half jq % 2 of the A fragment (mt, jq / 2) of
// P^T.  P[tok][tok'] = rq_tok rk_tok' e^{G_tok - G_tok'} q_tok . k_tok' for
// tok' <= tok, else 0, as in the output pass.
template <int DK>
struct PtHalf {
  int mt, jq;
  floatx4 acc;
  template <class SM>
  GDN_DEV void begin(const SM& C, int u, int lane) {
    mt = pt_half_mt(u);
    jq = pt_half_jq(u);
    acc = zero4();
    if (u < 10) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ks++)
        Mfma<bf16>::mma(acc, Mfma<bf16>::load_k8(C.q, SM::LDK, 16 * jq, 32 * ks, lane),
                        Mfma<bf16>::load_k8(C.k, SM::LDK, 16 * mt, 32 * ks, lane));
    }
  }
  template <class SM>
  GDN_DEV void finish(SM& C, int lane) const {
    const int g4 = lane >> 4, ln = lane & 15;
    const float* Gv = reinterpret_cast<const float*>(C.rec + kRecG);
    const int tokp = 16 * mt + ln, t0 = 16 * jq + 4 * g4;
    const float rkp = Gv[64 + tokp], Gp = Gv[tokp];
    const floatx4 rq4 = *reinterpret_cast<const floatx4*>(C.rq + t0);
    const floatx4 G4 = *reinterpret_cast<const floatx4*>(Gv + t0);
    bf16x4 f;
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const float val = acc[e] * rq4[e] * rkp * __expf(fminf(G4[e] - Gp, 0.f));
      f[e] = (bf16)(tokp <= t0 + e ? val : 0.f);
    }
    *reinterpret_cast<bf16x4*>(C.p + pt_frag(mt, jq >> 1) * 1024 + lane * 16 + (jq & 1) * 8) = f;
  }
};

template <int DK, int DV>
struct DsrCfg {
  static constexpr int CW = 32;          // dS columns a consumer wave
  static constexpr int NC = DV / CW;     // consumer waves
  static constexpr int NL = 4;           // loader waves
  static constexpr int NT = (NC + NL) * 64;
  typedef WsSmem<bf16, DK, DV, true> SM;
};

template <int DK, int DV>
__global__ __launch_bounds__((DsrCfg<DK, DV>::NT)) void dsr_kernel(BwdArgs a) {
  typedef DsrCfg<DK, DV> CF;
  typedef typename CF::SM SM;
  typedef Mfma<bf16> M;
  typedef M::frag Fr;
  constexpr int NC = CF::NC, NL = CF::NL, CW = CF::CW, NN = CW / 16;
  constexpr int KS = M::KSTEP, NSK = DK / KS, NSB = BT / KS, DKT = DK / 16;
  static_assert(KS == 32 && NSB == 2, "bf16 fragments of 64-token chunks");
  __shared__ SM buf[2];
  __shared__ unsigned p_count;  // loader waves' stored chunks (P^T hand-off)
  if (threadIdx.x == 0) p_count = 0u;
  __syncthreads();

  const int seg = blockIdx.x, h = blockIdx.y;
  if (seg >= a.counts[0]) return;
  const int4 ent = a.seg_table[seg];
  const int n = ent.x, Hv = a.Hv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, ln = lane & 15;
  const int64_t s0 = ent.y, e0 = ent.z;
  const int nch = (int)((e0 - s0 + BT - 1) / BT);
  const int chunk0 = a.seg_chunk0[seg];
  const bool replay = a.seq_rev_warm && a.seq_rev_warm[(int64_t)n * Hv + h];
  // a replaying sequence: the chunks after the segment run first (no dS'
  // stores), from zero or, reaching the sequence end, from dht
  int nwarm = 0;
  bool warm_dht = false;
  if (replay && !(ent.w & kLast)) {
    const int v = a.rev_warm[(int64_t)seg * Hv + h];
    nwarm = v & ~kWarmFromStart;
    warm_dht = (v & kWarmFromStart) != 0;
  }
  const int64_t te = nwarm > 0 ? (a.cu[n + 1] < a.T ? (int64_t)a.cu[n + 1] : a.T) : e0;
  const int nsteps = nch + nwarm;  // step i runs chunk nsteps - 1 - i
  const char* recs = a.rec + (int64_t)h * kRecBytes;
  const int64_t rstride = (int64_t)Hv * kRecBytes;

  if (wave >= NC) {
    // ======================= loaders =======================
    typedef WsLoad<bf16, DK, DV, true, SM::REC> LD;
    const int ltid = tid - NC * 64, lw = wave - NC;
    const int qa = h / (Hv / a.Hk);
    const bf16* qp = (const bf16*)a.q + (int64_t)qa * DK;
    const bf16* kp = (const bf16*)a.k + (int64_t)qa * DK;
    const bf16* op = (const bf16*)a.d_o + (int64_t)h * DV;
    const int64_t ld_o = (int64_t)Hv * DV;
    const typename LD::Off off = LD::offsets(a.ld_qk, ld_o, ltid);
    LD ld;
    if (nsteps > 0) {
      const int c = nsteps - 1;
      ld.load(qp, kp, a.ld_qk, op, ld_o, recs + (int64_t)(chunk0 + c) * rstride, s0 + (int64_t)c * BT,
              te, off, ltid);
    }
    for (int it = -1; it < nsteps; it++) {
      const int pc = it + 1;
      if (pc < nsteps) {
        SM& B = buf[pc & 1];
        ld.template store<true>(B, ltid, a.scale, a.use_l2norm);
        if (pc + 1 < nsteps) {
          const int c = nsteps - 2 - pc;
          ld.load(qp, kp, a.ld_qk, op, ld_o, recs + (int64_t)(chunk0 + c) * rstride,
                  s0 + (int64_t)c * BT, te, off, ltid);
        }
        // P^T and fo of the chunk just stored, once every loader wave's rows
        // are in place
        count_arrive(&p_count, lane);
        count_wait(&p_count, (unsigned)NL * (unsigned)(pc + 1));
        constexpr int NR = kPtHalves / NL;
        PtHalf<DK> ph[NR];
#pragma unroll
        for (int r = 0; r < NR; r++) ph[r].begin(B, lw + r * NL, lane);
#pragma unroll
        for (int r = 0; r < NR; r++) ph[r].finish(B, lane);
        if (lw == 0) B.fo[lane] = __expf(reinterpret_cast<const float*>(B.rec + kRecG)[lane]) * B.rq[lane];
      }
      lds_barrier();  // the chunk (with P^T, T^T and fo) is published
    }
    return;
  }

  // ======================= consumers =======================
  const int c0 = wave * CW;  // first dS column of this wave
  // dS tiles: rows dk_of_row(mt, 4(lane/16) + j), cols c0 + 16 nt + lane%16
  floatx4 dS[DKT][NN];
  {
    const float* dhtn = a.dht ? a.dht + ((int64_t)n * Hv + h) * DK * DV : nullptr;
    const float* src;
    if (nwarm > 0) src = warm_dht ? dhtn : nullptr;
    else if (!(ent.w & kLast)) src = a.seg_in + ((int64_t)seg * Hv + h) * DK * DV;
    else src = dhtn;
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          dS[mt][nt][j] = src ? src[dk_of_row(mt, 4 * g4 + j) * DV + c0 + 16 * nt + ln] : 0.f;
  }
  lds_barrier();  // the first chunk is published
  for (int i = 0; i < nsteps; i++) {
    SM& C = buf[i & 1];
    const int c = nsteps - 1 - i;
    if (c < nch) {
      // dS' of this chunk for the gradient kernel ([dk][dv], the activation
      // type): element stores through a buffer resource over it, the lane's
      // part of the offset (row 8 g4 of dk_of_row, its column) fixed
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc((bf16*)a.dstates + ((int64_t)(chunk0 + c) * Hv + h) * DK * DV,
                      (uint32_t)(DK * DV * sizeof(bf16)));
      const uint32_t soff = (uint32_t)((8 * g4 * DV + c0 + ln) * sizeof(bf16));
#pragma unroll
      for (int mt = 0; mt < DKT; mt++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++)
#pragma unroll
          for (int j = 0; j < 4; j++)
            buffer_store_elem<bf16>((bf16)dS[mt][nt][j], rs, soff,
                                    (uint32_t)(((32 * (mt >> 1) + 4 * (mt & 1) + j) * DV + 16 * nt) * sizeof(bf16)));
    }
    // x = k dS' (token rows), one contraction step of dS' at a time
    floatx4 x[4][NN];
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) x[mt][nt] = zero4();
#pragma unroll
    for (int s = 0; s < NSK; s++) {
      Fr b[NN];
#pragma unroll
      for (int nt = 0; nt < NN; nt++) b[nt] = acc_as_b<bf16>(dS, s, nt);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
        const Fr kf = M::load_k8(C.k, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(x[mt][nt], kf, b[nt]);
      }
    }
    const float* Fd = reinterpret_cast<const float*>(C.rec + kRecF);
    const float* Fk = Fd + 64;
    const float eC = Fd[128];
    // dx = fd o x + P^T dO (dO of this wave's columns as B fragments, token
    // rows in the convention's order)
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const floatx4 fd = *reinterpret_cast<const floatx4*>(Fd + 16 * mt + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NN; nt++) x[mt][nt] *= fd;
    }
    Fr dob[NSB][NN];
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) dob[s][nt] = M::load_col(C.v, SM::LDV, c0 + 16 * nt, s * KS, lane);
#pragma unroll
    for (int s = 0; s < NSB; s++)
#pragma unroll
      for (int mt = 0; mt < 2 + 2 * s; mt++) {
        const Fr pf = *reinterpret_cast<const Fr*>(C.p + pt_frag(mt, s) * 1024 + lane * 16);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(x[mt][nt], pf, dob[s][nt]);
      }
    // dy = T^T dx
    {
      Fr ys[NSB][NN];
#pragma unroll
      for (int s = 0; s < NSB; s++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++) ys[s][nt] = acc_as_b<bf16>(x, s, nt);
#pragma unroll
      for (int mt = 0; mt < 4; mt++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++) x[mt][nt] = zero4();
#pragma unroll
      for (int s = 0; s < NSB; s++)
#pragma unroll
        for (int mt = 0; mt < 2 + 2 * s; mt++) {
          const Fr tf = *reinterpret_cast<const Fr*>(C.rec + kRecT + pt_frag(mt, s) * 1024 + lane * 16);
#pragma unroll
          for (int nt = 0; nt < NN; nt++) M::mma(x[mt][nt], tf, ys[s][nt]);
        }
    }
    // dS <- eC dS' + q^T (fo o dO) - k^T (fk o dy)
    Fr bq[NSB][NN], bk[NSB][NN];
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      const floatx4 fk = *reinterpret_cast<const floatx4*>(Fk + 16 * mt + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NN; nt++) x[mt][nt] *= -fk;
    }
#pragma unroll
    for (int s = 0; s < NSB; s++) {
      const floatx4 flo = *reinterpret_cast<const floatx4*>(C.fo + s * KS + 4 * g4);
      const floatx4 fhi = *reinterpret_cast<const floatx4*>(C.fo + s * KS + 16 + 4 * g4);
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        bk[s][nt] = acc_as_b<bf16>(x, s, nt);
#pragma unroll
        for (int e = 0; e < 4; e++) {
          bq[s][nt][e] = (bf16)((float)dob[s][nt][e] * flo[e]);
          bq[s][nt][4 + e] = (bf16)((float)dob[s][nt][4 + e] * fhi[e]);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < DKT; mt++) {
      floatx4 acc[NN];
#pragma unroll
      for (int nt = 0; nt < NN; nt++) acc[nt] = dS[mt][nt] * eC;
      const int cdk = 32 * (mt >> 1) + 4 * (mt & 1);
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        const bf16x4 qlo = lds_rows4_tr(C.q, SM::LDK, s * KS, cdk, lane, 8);
        const bf16x4 qhi = lds_rows4_tr(C.q, SM::LDK, s * KS + 16, cdk, lane, 8);
        const Fr qf{qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        const bf16x4 klo = lds_rows4_tr(C.k, SM::LDK, s * KS, cdk, lane, 8);
        const bf16x4 khi = lds_rows4_tr(C.k, SM::LDK, s * KS + 16, cdk, lane, 8);
        const Fr kf{klo[0], klo[1], klo[2], klo[3], khi[0], khi[1], khi[2], khi[3]};
#pragma unroll
        for (int nt = 0; nt < NN; nt++) {
          M::mma(acc[nt], qf, bq[s][nt]);
          M::mma(acc[nt], kf, bk[s][nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NN; nt++) dS[mt][nt] = acc[nt];
    }
    lds_barrier();
  }
  // dh0 from a sequence's first segment
  if ((ent.w & kFirst) && a.dh0) {
    float* dst = a.dh0 + ((int64_t)n * Hv + h) * DK * DV;
#pragma unroll
    for (int mt = 0; mt < DKT; mt++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
#pragma unroll
        for (int j = 0; j < 4; j++) dst[dk_of_row(mt, 4 * g4 + j) * DV + c0 + 16 * nt + ln] = dS[mt][nt][j];
  }
}

// ---------------------------------------------------------------------------
// 3. local gradients of one (chunk, head)
// ---------------------------------------------------------------------------
template <typename E, int DK, int DV>
struct GradSmemCore {
  typedef Smem<E, DK, DV, true> SM;
  static constexpr int LDA = BT + 4;  // dA, dA^T, M1 + M1^T: [64][68] operand type
  static constexpr int NW = BwdCfg<E, DK, DV>::NW;
  static constexpr bool MS_IN_V = sizeof(E) * BT * SM::LDV >= sizeof(E) * BT * LDA;
  SM b;
  alignas(16) E dO[BT * SM::LDV];
  alignas(16) E ms_own[MS_IN_V ? 8 : BT * LDA];
  alignas(16) float part[4][NW][BT];  // row sums over each wave's columns
  alignas(16) float tp[5][4][BT];     // row/column sums of the 64x64 tiles
  alignas(16) float dot[NW];
  // one value head a q/k head: per-wave row sums of u_q . dq-hat and
  // u_k . dk-hat over each wave's key columns, and their totals (the l2norm
  // backward in place)
  alignas(16) float epi[2][NW][BT];
  alignas(16) float etot[2][BT];
};
// bfloat16, with room in LDS: dA gets its own array (else it goes over L,
// which the dL tiles read, and the dL and dP tiles run in two phases; the
// float32 kernels, short of registers, keep that form).
template <typename E, int DK, int DV>
struct GradSmem : GradSmemCore<E, DK, DV> {
  typedef GradSmemCore<E, DK, DV> Core;
  static constexpr bool DA_OWN =
      std::is_same<E, bf16>::value && sizeof(Core) + sizeof(E) * BT * Core::LDA + 256 <= 160 * 1024;
  alignas(16) E da_own[DA_OWN ? BT * Core::LDA : 8];
};

// row-partials kinds
enum { kRB = 0, kRYKS = 1, kRDOQS = 2, kRKDSVN = 3 };
// tile partial kinds
enum { kRowP = 0, kColP = 1, kRowKK = 2, kRowL = 3, kColL = 4 };

// sum over the 16 lanes of each lane group (one C-tile row)
GDN_DEV float row16_sum(float v) { return row_group_sum<16>(v); }

template <typename E, int DK, int DV>
__global__ __launch_bounds__((BwdCfg<E, DK, DV>::NT)) void grad_kernel(BwdArgs a) {
  static_assert(DK == DV, "the gradient kernel assumes dk == dv");
  typedef BwdCfg<E, DK, DV> CF;
  typedef typename CF::O O;
  typedef Mfma<O> M;
  typedef GradSmem<E, DK, DV> GS;
  typedef typename GS::SM SM;
  constexpr int NW = CF::NW, NT = CF::NT, KS = M::KSTEP;
  constexpr int NSK = DK / KS, NSB = BT / KS;
  constexpr int LDV = SM::LDV, LDA = GS::LDA;
  __shared__ GS gs;
  SM& sm = gs.b;

  const int c = blockIdx.x, h = blockIdx.y;
  if (c >= a.counts[1]) return;
  const int4 ent = a.chunk_tab[c];
  const int64_t tc = ent.x, te = ent.y;
  const int Hv = a.Hv, qa = h / (Hv / a.Hk);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, ln = lane & 15;
  constexpr int CW = CF::CW, NN = CW / 16;
  const int c0 = wave * CW;

  // bfloat16: T_r = (I + diag(beta) L)^-1 diag(beta) comes from the forward
  // prep's record (its six A fragments, scattered into a row-major bf16 copy
  // Trm over Tm's space) instead of a solve here; then T = I - T_r L
  constexpr bool REC_T = std::is_same<E, bf16>::value;
  static_assert(!REC_T || uses_prep<E, DK, DV, kStates>(), "bfloat16 keeps the prep's records");
  O* const Trm = reinterpret_cast<O*>(sm.Tm);
  constexpr int LDT = SM::LDT;
  static_assert(sizeof(O) * BT * LDT <= sizeof(sm.Tm), "T_r copy within Tm");

  zero_upper<O, true, NT>(sm, tid);
  {
    typename CF::PF pf;
    pf.load((const E*)a.q + (int64_t)qa * DK, (const E*)a.k + (int64_t)qa * DK, a.ld_qk,
            (const E*)a.v + (int64_t)h * DV, a.ld_v, a.g + h, a.beta + h, Hv, tc, te, tid);
    constexpr int TRV = 6 * 64, TRP = (TRV + NT - 1) / NT;  // record vectors of T_r
    bf16x8 trv[TRP];
    if constexpr (REC_T) {
      const char* R = a.rec + ((int64_t)c * Hv + h) * kRecBytes + kRecT;
#pragma unroll
      for (int p = 0; p < TRP; p++) {
        const int i = tid + NT * p;
        if (i < TRV) trv[p] = *reinterpret_cast<const bf16x8*>(R + 16 * i);
      }
    }
    typedef typename Vec16<E>::type V16;
    constexpr int VE = Vec16<E>::N, VPR = DV / VE;
    // dO rows: every vector of the thread loaded (from a valid row: past the
    // sequence end the chunk's first, zeroed after) before any is stored, so
    // the loads are in flight together
    const E* dop = (const E*)a.d_o + (int64_t)h * DV;
    constexpr int DOP = (BT * VPR + NT - 1) / NT;
    V16 dov[DOP];
#pragma unroll
    for (int p = 0; p < DOP; p++) {
      const int i = tid + NT * p;
      const int64_t t = tc + i / VPR;
      const bool ok = i < BT * VPR && t < te;
      dov[p] = *reinterpret_cast<const V16*>(dop + ((ok ? t : tc) * Hv) * DV + (ok ? i % VPR : 0) * VE);
    }
#pragma unroll
    for (int p = 0; p < DOP; p++) {
      const int i = tid + NT * p;
      if (i < BT * VPR)
        *reinterpret_cast<V16*>(gs.dO + (i / VPR) * LDV + (i % VPR) * VE) =
            tc + i / VPR < te ? dov[p] : zero_vec16<E>();
    }
    stage<E, O, DK, DV, NT, true>(sm, pf, a.scale, a.use_l2norm, tid);
    if constexpr (REC_T) {
      // vector i: fragment p_frag(mt, s) = i / 64, lane l = i % 64, elements
      // T_r[16 mt + l%16][32 s + 16 h + 4(l/16) + e], h = 0, 1, e = 0..3
#pragma unroll
      for (int p = 0; p < TRP; p++) {
        const int i = tid + NT * p;
        if (i < TRV) {
          const int fp = i >> 6, l = i & 63;
          const int mt = fp < 2 ? fp : (fp + 2) >> 1, s2 = fp < 2 ? 0 : (fp & 1);
          O* dst = Trm + (16 * mt + (l & 15)) * LDT + 32 * s2 + 4 * (l >> 4);
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{trv[p][0], trv[p][1], trv[p][2], trv[p][3]};
          *reinterpret_cast<bf16x4*>(dst + 16) = bf16x4{trv[p][4], trv[p][5], trv[p][6], trv[p][7]};
        }
      }
    }
  }
  __syncthreads();
  floatx4 vn[4][NN];
  if constexpr (REC_T) {
    // L and P tiles; u = T_r v (this wave's columns); W = T_r diag(e^G) kh
    for (int t = wave; t < 20; t += NW) {
      int ti, tj;
      lower_tile_ij(t % 10, ti, tj);
      gram_tile<O, DK>(sm, t >= 10, ti, tj, lane);
    }
    {
      typename M::frag b[NSB][NN];
#pragma unroll
      for (int s = 0; s < NSB; s++)
#pragma unroll
        for (int nt = 0; nt < NN; nt++) b[s][nt] = M::load_col(sm.v, LDV, c0 + 16 * nt, s * KS, lane);
#pragma unroll
      for (int mt = 0; mt < 4; mt++) {
#pragma unroll
        for (int nt = 0; nt < NN; nt++) vn[mt][nt] = zero4();
#pragma unroll
        for (int s = 0; s < NSB; s++)
          if (2 * s <= mt) {  // the fragments right of the diagonal are zero
            const typename M::frag tf = M::load(Trm, LDT, 16 * mt, s * KS, lane);
#pragma unroll
            for (int nt = 0; nt < NN; nt++) M::mma(vn[mt][nt], tf, b[s][nt]);
          }
      }
    }
    {
      constexpr int NTILE = 4 * (DK / 16);
      for (int tt = wave; tt < NTILE; tt += NW) {
        const int mt = tt % 4, nt = tt / 4;
        floatx4 acc = zero4();
#pragma unroll
        for (int s = 0; s < NSB; s++)
          if (2 * s <= mt)
            M::mma(acc, M::load(Trm, LDT, 16 * mt, s * KS, lane),
                   M::load_col_scaled(sm.k, SM::LDK, 16 * nt, s * KS, sm.eg, lane));
        const int rb = 16 * mt + 4 * g4, cc = 16 * nt + ln;
#pragma unroll
        for (int jj = 0; jj < 4; jj++) sm.w[(rb + jj) * SM::LDK + cc] = from_f<O>(acc[jj]);
      }
    }
  } else {
    gram_kk<O, DK, NW>(sm, wave, lane);
    __syncthreads();
    solve<O, DK, NW, true>(sm, wave, lane);
    compute_u<O, NN>(sm, c0, lane, vn);  // u, turned into Vn below
    compute_w<O, DK, NW>(sm, wave, lane);
  }
  __syncthreads();

  const float GC = sm.G[BT - 1];
  const E* Sg = (const E*)a.states + ((int64_t)c * Hv + h) * DK * DV;
  const E* dSg = (const E*)a.dstates + ((int64_t)c * Hv + h) * DK * DV;

  // S and dS' as B fragments (K = dk, N = this wave's value columns) and <dS', S>
  typename M::frag sb[NSK][NN], dsb[NSK][NN];
  float dot = 0.f;
  if constexpr (sizeof(E) == 2) {
    // 16-bit element loads through buffer resources over the two tiles: the
    // lane's part of the offset (row 4 g4, its column) is fixed and the rest
    // constant, so there is no address arithmetic and the halves go straight
    // into the fragment registers.  <dS', S> over this wave's columns is the
    // trace of S^T dS' (four products; the diagonal entry of a lane is its
    // element j = ln % 4 when g4 = ln / 4).
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(Sg, (uint32_t)(DK * DV * sizeof(E)));
    const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(dSg, (uint32_t)(DK * DV * sizeof(E)));
    const uint32_t voff = (uint32_t)((4 * g4 * DV + c0 + ln) * sizeof(E));
    floatx4 tr = zero4();
#pragma unroll
    for (int s = 0; s < NSK; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const uint32_t soff = (uint32_t)(((32 * s + 16 * (e >> 2) + (e & 3)) * DV + 16 * nt) * sizeof(E));
          sb[s][nt][e] = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0));
          dsb[s][nt][e] = __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(rd, voff, soff, 0));
        }
        M::mma(tr, sb[s][nt], dsb[s][nt]);
      }
#pragma unroll
    for (int j = 0; j < 4; j++) dot += (4 * g4 + j == ln) ? tr[j] : 0.f;
  } else {
    // fp32 states: one C tile a contraction step, element loads
    static_assert(KS == 16, "fp32 contraction step");
#pragma unroll
    for (int s = 0; s < NSK; s++)
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        floatx4 st, dt;
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int idx = (16 * s + 4 * g4 + j) * DV + c0 + 16 * nt + ln;
          st[j] = to_f(Sg[idx]);
          dt[j] = to_f(dSg[idx]);
          dot += st[j] * dt[j];
        }
        sb[s][nt] = M::from_acc(st);
        dsb[s][nt] = M::from_acc(dt);
      }
  }

  // Vn = u - W S; QS; KS; K dS'
  floatx4 ks[4][NN], kds[4][NN];
  float r_doqs[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    floatx4 wq[NN], qq[NN], kq[NN], dq[NN];
#pragma unroll
    for (int nt = 0; nt < NN; nt++) wq[nt] = qq[nt] = kq[nt] = dq[nt] = zero4();
#pragma unroll
    for (int s = 0; s < NSK; s++) {
      const typename M::frag wf = M::load(sm.w, SM::LDK, 16 * mt, s * KS, lane);
      const typename M::frag qf = M::load(sm.q, SM::LDK, 16 * mt, s * KS, lane);
      const typename M::frag kf = M::load(sm.k, SM::LDK, 16 * mt, s * KS, lane);
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        M::mma(wq[nt], wf, sb[s][nt]);
        M::mma(qq[nt], qf, sb[s][nt]);
        M::mma(kq[nt], kf, sb[s][nt]);
        M::mma(dq[nt], kf, dsb[s][nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NN; nt++) {
      vn[mt][nt] -= wq[nt];
      ks[mt][nt] = kq[nt];
      kds[mt][nt] = dq[nt];
    }
    // dO tiles (mt, this wave's columns) in C layout
#pragma unroll
    for (int j = 0; j < 4; j++) r_doqs[mt][j] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NN; nt++) {
      const floatx4 o = lds_tile_c(gs.dO, LDV, 16 * mt, c0 + 16 * nt, lane);
#pragma unroll
      for (int j = 0; j < 4; j++) r_doqs[mt][j] += o[j] * qq[nt][j];
    }
  }
  // dVn = P^T dO + D o K dS'
  floatx4 dvn[4][NN];
  float r_kdsvn[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    floatx4 pp[NN];
#pragma unroll
    for (int nt = 0; nt < NN; nt++) pp[nt] = zero4();
#pragma unroll
    for (int s = 0; s < NSB; s++) {
      const typename M::frag pt = M::load_col(sm.p, SM::LDT, 16 * mt, s * KS, lane);
#pragma unroll
      for (int nt = 0; nt < NN; nt++)
        M::mma(pp[nt], pt, M::load_col(gs.dO, LDV, c0 + 16 * nt, s * KS, lane));
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int row = 16 * mt + 4 * g4 + j;
      const float d = __expf(GC - sm.G[row]);
      r_kdsvn[mt][j] = 0.f;
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        r_kdsvn[mt][j] += kds[mt][nt][j] * vn[mt][nt][j];
        pp[nt][j] += d * kds[mt][nt][j];
      }
    }
#pragma unroll
    for (int nt = 0; nt < NN; nt++) dvn[mt][nt] = pp[nt];
  }
  // Y = T^T dVn; dv = beta o Y (bfloat16: dv = T_r^T dVn, then Y = dVn -
  // L^T dv, since T = I - T_r L)
  floatx4 dvr[REC_T ? 4 : 1][NN];
  if constexpr (REC_T) {
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
#pragma unroll
      for (int nt = 0; nt < NN; nt++) dvr[mt][nt] = zero4();
#pragma unroll
      for (int s = 0; s < NSB; s++)
        if (mt < 2 + 2 * s) {  // the fragments left of the diagonal are zero
          const typename M::frag tt = M::load_col(Trm, LDT, 16 * mt, s * KS, lane);
#pragma unroll
          for (int nt = 0; nt < NN; nt++) M::mma(dvr[mt][nt], tt, acc_as_b<O>(dvn, s, nt));
        }
    }
  }
  floatx4 y[4][NN];
  float r_b[4][4], r_yks[4][4];
  // dv, dq and dk rows of this chunk through buffer resources (rows past the
  // sequence end fall outside the range and their stores are dropped); the
  // lane's part of the offset (row 4 g4, its column) is fixed
  const int64_t nrows = te - tc;
  const __amdgpu_buffer_rsrc_t rdv =
      buffer_rsrc((E*)a.dv + tc * a.ld_dv + (int64_t)h * DV,
                  (uint32_t)(((nrows - 1) * a.ld_dv + DV) * (int64_t)sizeof(E)));
  const uint32_t dvoff = (uint32_t)((4 * g4 * a.ld_dv + c0 + ln) * (int64_t)sizeof(E));
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    floatx4 yy[NN];
    if constexpr (REC_T) {
#pragma unroll
      for (int nt = 0; nt < NN; nt++) yy[nt] = dvn[mt][nt];
#pragma unroll
      for (int s = 0; s < NSB; s++)
        if (mt < 2 + 2 * s) {
          typename M::frag lt = M::load_col_f32(sm.L, SM::LDF, 16 * mt, s * KS, nullptr, lane);
#pragma unroll
          for (int e = 0; e < 8; e++) lt[e] = -lt[e];  // -L^T
#pragma unroll
          for (int nt = 0; nt < NN; nt++) M::mma(yy[nt], lt, acc_as_b<O>(dvr, s, nt));
        }
    } else {
#pragma unroll
      for (int nt = 0; nt < NN; nt++) yy[nt] = zero4();
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        const typename M::frag tt = M::load_col_f32(sm.Tm, SM::LDF, 16 * mt, s * KS, nullptr, lane);
#pragma unroll
        for (int nt = 0; nt < NN; nt++) M::mma(yy[nt], tt, acc_as_b<O>(dvn, s, nt));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) r_b[mt][j] = r_yks[mt][j] = 0.f;
#pragma unroll
    for (int nt = 0; nt < NN; nt++) {
      y[mt][nt] = yy[nt];
      const floatx4 vv = lds_tile_c(sm.v, LDV, 16 * mt, c0 + 16 * nt, lane);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 16 * mt + 4 * g4 + j;
        r_b[mt][j] += yy[nt][j] * vv[j];
        r_yks[mt][j] += yy[nt][j] * ks[mt][nt][j];
        const float dvj = REC_T ? dvr[REC_T ? mt : 0][nt][j] : sm.beta[row] * yy[nt][j];
        buffer_store_elem<E>(from_f<E>(dvj), rdv, dvoff,
                             (uint32_t)(((16 * mt + j) * a.ld_dv + 16 * nt) * (int64_t)sizeof(E)));
      }
    }
  }
  // row sums over this wave's columns
  dot = wave_sum(dot);
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float v0 = row16_sum(r_b[mt][j]), v1 = row16_sum(r_yks[mt][j]),
                  v2 = row16_sum(r_doqs[mt][j]), v3 = row16_sum(r_kdsvn[mt][j]);
      if (ln == 0) {
        const int row = 16 * mt + 4 * g4 + j;
        gs.part[kRB][wave][row] = v0;
        gs.part[kRYKS][wave][row] = v1;
        gs.part[kRDOQS][wave][row] = v2;
        gs.part[kRKDSVN][wave][row] = v3;
      }
    }
  if (lane == 0) gs.dot[wave] = dot;
  __syncthreads();  // w, Tm, v, p-columns reads done
  // Vn over w, Y over Tm (operand type, [64][LDV])
  O* sVn = sm.w;
  O* sY = reinterpret_cast<O*>(sm.Tm);
#pragma unroll
  for (int mt = 0; mt < 4; mt++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int row = 16 * mt + 4 * g4 + j;
#pragma unroll
      for (int nt = 0; nt < NN; nt++) {
        sVn[row * LDV + c0 + 16 * nt + ln] = from_f<O>(vn[mt][nt][j]);
        sY[row * LDV + c0 + 16 * nt + ln] = from_f<O>(y[mt][nt][j]);
      }
    }
  __syncthreads();

  // the key side's S and dS' fragments (B[k = value idx][n = key idx] =
  // S[n][k]), loaded here so that they arrive during the dL and dP tiles
  typename M::frag kst[NN][NSK], kdst[NN][NSK];
#pragma unroll
  for (int nt = 0; nt < NN; nt++)
#pragma unroll
    for (int s = 0; s < NSK; s++) {
      kst[nt][s] = M::load(Sg, DV, c0 + 16 * nt, s * KS, lane);
      kdst[nt][s] = M::load(dSg, DV, c0 + 16 * nt, s * KS, lane);
    }
  // dL = -Y Vn^T (strict lower): M1 + M1^T, dbeta and dG partials
  O* sMs = GS::MS_IN_V ? sm.v : gs.ms_own;
  auto dl_tile = [&](int t) {
    int i, j;
    lower_tile_ij(t, i, j);
    floatx4 acc = zero4();
#pragma unroll
    for (int s = 0; s < DV / KS; s++)
      M::mma(acc, M::load(sY, LDV, 16 * i, s * KS, lane), M::load(sVn, LDV, 16 * j, s * KS, lane));
    const int col = 16 * j + ln;
    float rk[4], rl[4], cl = 0.f;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int row = 16 * i + 4 * g4 + jj;
      const bool lo = row > col;
      const float dl = lo ? -acc[jj] : 0.f;
      const float kk = sm.L[row * SM::LDF + col];  // kh.kh o Gamma (strict lower, no beta)
      const float gam = lo ? __expf(sm.G[row] - sm.G[col]) : 0.f;
      const float m1 = sm.beta[row] * dl * gam;
      rk[jj] = dl * kk;
      rl[jj] = dl * sm.beta[row] * kk;
      cl += rl[jj];
      if (i > j || lo) {
        sMs[row * LDA + col] = from_f<O>(m1);
        sMs[col * LDA + row] = from_f<O>(m1);
      } else if (row == col) {
        sMs[row * LDA + col] = from_f<O>(0.f);
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const float a1 = row16_sum(rk[jj]), a2 = row16_sum(rl[jj]);
      if (ln == 0) {
        gs.tp[kRowKK][j][16 * i + 4 * g4 + jj] = a1;
        gs.tp[kRowL][j][16 * i + 4 * g4 + jj] = a2;
      }
    }
    cl = rows4_sum(cl);
    if (g4 == 0) gs.tp[kColL][i][col] = cl;
  };
  // dP = dO Vn^T (lower incl): dA = dP o Gamma; dG partials
  O* sdA = GS::DA_OWN ? gs.da_own : reinterpret_cast<O*>(sm.L);
  auto dp_tile = [&](int t) -> floatx4 {
    int i, j;
    lower_tile_ij(t, i, j);
    floatx4 acc = zero4();
#pragma unroll
    for (int s = 0; s < DV / KS; s++)
      M::mma(acc, M::load(gs.dO, LDV, 16 * i, s * KS, lane), M::load(sVn, LDV, 16 * j, s * KS, lane));
    const int col = 16 * j + ln;
    float rp[4], cp = 0.f;
    floatx4 da;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int row = 16 * i + 4 * g4 + jj;
      const bool lo = row >= col;
      const float dp = lo ? acc[jj] : 0.f;
      da[jj] = lo ? dp * __expf(sm.G[row] - sm.G[col]) : 0.f;
      rp[jj] = dp * to_f(sm.p[row * SM::LDT + col]);
      cp += rp[jj];
      sdA[row * LDA + col] = from_f<O>(da[jj]);
      if (i > j) sdA[(16 * j + 4 * g4 + jj) * LDA + 16 * i + ln] = from_f<O>(0.f);
    }
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const float a1 = row16_sum(rp[jj]);
      if (ln == 0) gs.tp[kRowP][j][16 * i + 4 * g4 + jj] = a1;
    }
    cp = rows4_sum(cp);
    if (g4 == 0) gs.tp[kColP][i][col] = cp;
    return da;
  };
  // the dP tiles of this wave (tile index, dA values) for dA^T below
  constexpr int NDP = GS::DA_OWN ? (20 + NW - 1) / NW : (10 + NW - 1) / NW;
  floatx4 dat[NDP];
  int dpt[NDP];
  int nmine = 0;
  if constexpr (GS::DA_OWN) {
    // the dL and dP tiles in one phase (dA does not go over L)
    for (int t = wave; t < 20; t += NW) {
      if (t < 10) {
        dl_tile(t);
      } else {
        dat[nmine] = dp_tile(t - 10);
        dpt[nmine++] = t - 10;
      }
    }
  } else {
    for (int t = wave; t < 10; t += NW) dl_tile(t);
    __syncthreads();  // L reads done: dA goes over L
    for (int t = wave; t < 10; t += NW) {
      dat[nmine] = dp_tile(t);
      dpt[nmine++] = t;
    }
  }
  __syncthreads();  // P reads done: dA^T goes over p
  O* sdAT = sm.p;
  for (int m = 0; m < nmine; m++) {
    int i, j;
    lower_tile_ij(dpt[m], i, j);
    const int col = 16 * j + ln;
#pragma unroll
    for (int jj = 0; jj < 4; jj++) {
      const int row = 16 * i + 4 * g4 + jj;
      sdAT[col * LDA + row] = from_f<O>(dat[m][jj]);
      if (i > j) sdAT[(16 * i + 4 * g4 + jj) * LDA + 16 * j + ln] = from_f<O>(0.f);
    }
  }
  __syncthreads();

  // dk-side: this wave's key columns [c0, c0 + CW).  With one value head a
  // q/k head there is nothing to sum over heads, so the l2norm backward runs
  // here (fused) and dq, dk are written directly; otherwise dq-hat, dk-hat go
  // to the fp32 partials for finalize_qk_kernel.
  const bool fused = a.Hv == a.Hk;
  // fp32 partial rows [token][Hv][2][dk] of this chunk and head (a buffer
  // resource: rows past the sequence end are dropped)
  const __amdgpu_buffer_rsrc_t rqk =
      buffer_rsrc(a.dqk + (tc * Hv + h) * 2 * DK,
                  (uint32_t)(((nrows - 1) * Hv * 2 * DK + 2 * DK) * (int64_t)sizeof(float)));
  const uint32_t qkoff = (uint32_t)((4 * g4 * Hv * 2 * DK + ln) * (int64_t)sizeof(float));
  float fq[NN][4][4], fk[NN][4][4];
#pragma unroll
  for (int nt = 0; nt < NN; nt++) {
    const int dc = c0 + 16 * nt;
    typename M::frag st[NSK], dst[NSK], kc[NSB], qc[NSB];
#pragma unroll
    for (int s = 0; s < NSK; s++) {
      st[s] = kst[nt][s];
      dst[s] = kdst[nt][s];
    }
#pragma unroll
    for (int s = 0; s < NSB; s++) {
      kc[s] = M::load_col(sm.k, SM::LDK, dc, s * KS, lane);
      qc[s] = M::load_col(sm.q, SM::LDK, dc, s * KS, lane);
    }
#pragma unroll
    for (int mt = 0; mt < 4; mt++) {
      floatx4 a1 = zero4(), a2 = zero4(), b3 = zero4(), b4 = zero4(), b5 = zero4(), b6 = zero4();
#pragma unroll
      for (int s = 0; s < NSK; s++) {
        M::mma(a1, M::load(gs.dO, LDV, 16 * mt, s * KS, lane), st[s]);
        M::mma(b4, M::load(sVn, LDV, 16 * mt, s * KS, lane), dst[s]);
        M::mma(b5, M::load(sY, LDV, 16 * mt, s * KS, lane), st[s]);
      }
#pragma unroll
      for (int s = 0; s < NSB; s++) {
        M::mma(a2, M::load(sdA, LDA, 16 * mt, s * KS, lane), kc[s]);
        M::mma(b3, M::load(sdAT, LDA, 16 * mt, s * KS, lane), qc[s]);
        M::mma(b6, M::load(sMs, LDA, 16 * mt, s * KS, lane), kc[s]);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 16 * mt + 4 * g4 + j;
        const float gm = sm.eg[row];
        const float d = __expf(GC - sm.G[row]);
        const float dqv = gm * a1[j] + a2[j];
        const float dkv = b3[j] + d * b4[j] - sm.beta[row] * gm * b5[j] + b6[j];
        fq[nt][mt][j] = dqv;
        fk[nt][mt][j] = dkv;
        if (!fused) {
          const uint32_t so = (uint32_t)(((16 * mt + j) * Hv * 2 * DK + dc) * sizeof(float));
          buffer_store_elem<float>(dqv, rqk, qkoff, so);
          buffer_store_elem<float>(dkv, rqk, qkoff, so + (uint32_t)(DK * sizeof(float)));
        }
      }
    }
  }
  if (fused) {
    // the unit rows u = q-hat / scale and k-hat of this wave's columns (staged
    // in LDS) give dq = scale r_q (dq-hat - u (u . dq-hat)) and dk = r_k
    // (dk-hat - u_k (u_k . dk-hat)); the row dots are summed over the waves
    const float inv_scale = 1.f / a.scale;
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 16 * mt + 4 * g4 + j;
        float sqd = 0.f, skd = 0.f;
#pragma unroll
        for (int nt = 0; nt < NN; nt++) {
          const int col = c0 + 16 * nt + ln;
          sqd += to_f(sm.q[row * SM::LDK + col]) * inv_scale * fq[nt][mt][j];
          skd += to_f(sm.k[row * SM::LDK + col]) * fk[nt][mt][j];
        }
        sqd = row16_sum(sqd);
        skd = row16_sum(skd);
        if (ln == 0) {
          gs.epi[0][wave][row] = sqd;
          gs.epi[1][wave][row] = skd;
        }
      }
    __syncthreads();
    for (int i = tid; i < 2 * BT; i += NT) {
      const int kind = i / BT, row = i % BT;
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; w++) acc += gs.epi[kind][w][row];
      gs.etot[kind][row] = acc;
    }
    __syncthreads();
    const uint32_t span = (uint32_t)(((nrows - 1) * a.ld_dqk + DK) * (int64_t)sizeof(E));
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc((E*)a.dq + tc * a.ld_dqk + (int64_t)qa * DK, span);
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((E*)a.dk + tc * a.ld_dqk + (int64_t)qa * DK, span);
    const uint32_t qoff = (uint32_t)((4 * g4 * a.ld_dqk + c0 + ln) * (int64_t)sizeof(E));
#pragma unroll
    for (int mt = 0; mt < 4; mt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int row = 16 * mt + 4 * g4 + j;
        const float nq = sm.rnq[row], nk = sm.rnk[row];
        const float qd = gs.etot[0][row], kd = gs.etot[1][row];
#pragma unroll
        for (int nt = 0; nt < NN; nt++) {
          const int col = c0 + 16 * nt + ln;
          float gq = a.scale * fq[nt][mt][j], gk = fk[nt][mt][j];
          if (a.use_l2norm) {
            gq = a.scale * nq * (fq[nt][mt][j] - to_f(sm.q[row * SM::LDK + col]) * inv_scale * qd);
            gk = nk * (fk[nt][mt][j] - to_f(sm.k[row * SM::LDK + col]) * kd);
          }
          const uint32_t so = (uint32_t)(((16 * mt + j) * a.ld_dqk + 16 * nt) * (int64_t)sizeof(E));
          buffer_store_elem<E>(from_f<E>(gq), rq, qoff, so);
          buffer_store_elem<E>(from_f<E>(gk), rk, qoff, so);
        }
      }
  }

  // dbeta, dG -> dg (wave 0, lane = row)
  if (wave == 0) {
    const int r = lane;
    const int rb = r >> 4;
    float rB = 0.f, rYKS = 0.f, rDOQS = 0.f, rKDSVN = 0.f, dotS = 0.f;
#pragma unroll
    for (int w = 0; w < NW; w++) {
      rB += gs.part[kRB][w][r];
      rYKS += gs.part[kRYKS][w][r];
      rDOQS += gs.part[kRDOQS][w][r];
      rKDSVN += gs.part[kRKDSVN][w][r];
      dotS += gs.dot[w];
    }
    float rowP = 0.f, colP = 0.f, rowKK = 0.f, rowL = 0.f, colL = 0.f;
    for (int j = 0; j <= rb; j++) {
      rowP += gs.tp[kRowP][j][r];
      rowKK += gs.tp[kRowKK][j][r];
      rowL += gs.tp[kRowL][j][r];
    }
    for (int i = rb; i < 4; i++) {
      colP += gs.tp[kColP][i][r];
      colL += gs.tp[kColL][i][r];
    }
    const float gm = sm.eg[r], bt = sm.beta[r];
    const float d = __expf(GC - sm.G[r]);
    const float dbeta = rB - gm * rYKS + rowKK;
    float dG = gm * rDOQS - d * rKDSVN - bt * gm * rYKS + rowP - colP + rowL - colL;
    const float tail = wave_sum(d * rKDSVN) + __expf(GC) * dotS;  // d/dG_C terms
    if (r == BT - 1) dG += tail;
    // dg_t = sum_{s >= t} dG_s within the chunk: a prefix scan of the rows
    // in reverse order
    const float suf = __shfl(wave_incl_scan(__shfl(dG, BT - 1 - r, 64)), BT - 1 - r, 64);
    const int64_t t = tc + r;
    if (t < te) {
      a.dbeta[t * Hv + h] = dbeta;
      a.dg[t * Hv + h] = suf;
    }
  }
}

// ---------------------------------------------------------------------------
// 4. sum over value heads and back through l2norm / scale
// ---------------------------------------------------------------------------
template <typename E, int DK>
__global__ __launch_bounds__(256) void finalize_qk_kernel(BwdArgs a, int64_t units) {
  // a lane owns 4 consecutive elements (one 16-byte read of each fp32 partial
  // row), DK / 4 lanes a (token, q/k head) unit, 64 / (DK / 4) units a wave
  constexpr int LPU = DK / 4, UPW = 64 / LPU;
  static_assert(DK % 4 == 0 && LPU <= 64 && 64 % LPU == 0, "dk / 4 must divide 64");
  const int lane = threadIdx.x & 63, d0 = 4 * (lane % LPU);
  const int64_t u = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * UPW + lane / LPU;
  // a whole lane group is in or out of range: no lane leaves before the
  // group sums below
  const bool valid = u < units;
  const int64_t t = valid ? u / a.Hk : 0;
  const int qa = valid ? (int)(u % a.Hk) : 0;
  const int grp = a.Hv / a.Hk;
  float dq[4], dk[4], q[4], k[4];
  float qs = 0.f, ks = 0.f, qd = 0.f, kd = 0.f;
  const E* qp = (const E*)a.q + t * a.ld_qk + (int64_t)qa * DK + d0;
  const E* kp = (const E*)a.k + t * a.ld_qk + (int64_t)qa * DK + d0;
#pragma unroll
  for (int e = 0; e < 4; e++) dq[e] = dk[e] = q[e] = k[e] = 0.f;
  if (valid) {
    for (int hh = qa * grp; hh < (qa + 1) * grp; hh++) {
      const float* src = a.dqk + (t * a.Hv + hh) * 2 * DK + d0;
      const floatx4 vq = *reinterpret_cast<const floatx4*>(src);
      const floatx4 vk = *reinterpret_cast<const floatx4*>(src + DK);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        dq[e] += vq[e];
        dk[e] += vk[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; e++) {
      q[e] = to_f(qp[e]);
      k[e] = to_f(kp[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; e++) {
    qs += q[e] * q[e];
    ks += k[e] * k[e];
    qd += q[e] * dq[e];
    kd += k[e] * dk[e];
  }
  qs = group_sum<LPU>(qs);
  ks = group_sum<LPU>(ks);
  qd = group_sum<LPU>(qd);
  kd = group_sum<LPU>(kd);
  E* dqp = (E*)a.dq + t * a.ld_dqk + (int64_t)qa * DK + d0;
  E* dkp = (E*)a.dk + t * a.ld_dqk + (int64_t)qa * DK + d0;
  const float rq = a.use_l2norm ? 1.f / sqrtf(qs + 1e-6f) : 1.f;
  const float rk = a.use_l2norm ? 1.f / sqrtf(ks + 1e-6f) : 1.f;
  if (valid) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      float gq = a.scale * dq[e], gk = dk[e];
      if (a.use_l2norm) {
        gq = a.scale * rq * (dq[e] - q[e] * rq * rq * qd);
        gk = rk * (dk[e] - k[e] * rk * rk * kd);
      }
      dqp[e] = from_f<E>(gq);
      dkp[e] = from_f<E>(gk);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BwdLayout {
  Plan plan;
  size_t off_states, off_dstates, off_dqk, off_rev_warm, off_seq_rev_warm, end;
};

BwdLayout bwd_layout(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, gdn_dtype dt) {
  BwdLayout L;
  L.plan = make_plan(T, N, Hv, dk, dv, gdn::chunk_rec_bytes(dt));
  size_t o = L.plan.end;
  const size_t es = dt == GDN_BF16 ? 2 : 4;  // states in the activation type
  const size_t st = es * (size_t)L.plan.chunk_cap * Hv * dk * dv;
  L.off_states = o;
  o = gdn::round_up(o + st, 256);
  L.off_dstates = o;
  o = gdn::round_up(o + st, 256);
  L.off_dqk = o;
  o = gdn::round_up(o + sizeof(float) * (size_t)T * Hv * 2 * dk, 256);
  L.off_rev_warm = o;
  o = gdn::round_up(o + 4 * (size_t)L.plan.seg_cap * Hv, 256);
  L.off_seq_rev_warm = o;
  o = gdn::round_up(o + 4 * (size_t)N * Hv, 256);
  L.end = o;
  return L;
}

// saved: the buffer of a saving forward (gdn_chunk_fwd_save) on the same
// inputs, holding the records and the state entering every chunk; then the
// forward pipeline is not run again, only its plan.
template <typename E, int DK, int DV>
int launch_bwd(BwdArgs b, const LoopArgs& la_in, int N, int64_t T, const BwdLayout& L, char* ws,
               const char* saved, hipStream_t stream) {
  typedef BwdCfg<E, DK, DV> CF;
  // a saving forward writes records exactly when this backward reads them
  static_assert(!std::is_same<E, bf16>::value ||
                    uses_prep<E, DK, DV, kStates>() == uses_prep<E, DK, DV, kOut>(),
                "records of the forward and the backward");
  PlanPtrs pp = L.plan.ptrs(ws, true);
  b.counts = pp.counts;
  b.chunk_tab = pp.chunk_tab;
  b.seq_chunk_off = pp.seq_chunk_off;
  b.dstates = ws + L.off_dstates;
  b.dqk = reinterpret_cast<float*>(ws + L.off_dqk);
  if (saved) {
    const gdn::SavedLayout SL = gdn::chunk_saved_layout(T, N, b.Hv, DK, DV, std::is_same<E, bf16>::value ? GDN_BF16 : GDN_F32);
    b.states = saved + SL.off_states;
    b.rec = uses_prep<E, DK, DV, kStates>() ? saved + SL.off_rec : nullptr;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, b.cu, N, T, (int)L.plan.seg_first,
                       (int)L.plan.seg_len, (int)L.plan.seg_cap, (int)L.plan.chunk_cap, pp);
    if (int rc = gdn::check_launch("gdn_chunk_bwd(plan)")) return rc;
  } else {
    b.states = ws + L.off_states;
    LoopArgs la = la_in;
    la.states = ws + L.off_states;
    if (int rc = run_pipeline<E, DK, DV, kStates>(la, b.cu, N, T, L.plan, ws, true, stream)) return rc;
    b.rec = uses_prep<E, DK, DV, kStates>() ? ws + L.plan.off_rec : nullptr;
  }
  // dS pass over the forward's segments (its summary and initial-state buffers
  // are free again): reverse summaries, reverse scan from dht, final pass
  b.seg_table = pp.table;
  b.seg_chunk0 = pp.seg_chunk0;
  if (L.plan.split && b.rec) {
    // per (sequence, head): replay the dS recurrence instead of summaries
    // where the records' bounds allow it
    int32_t* rw = reinterpret_cast<int32_t*>(ws + L.off_rev_warm);
    int32_t* srw = reinterpret_cast<int32_t*>(ws + L.off_seq_rev_warm);
    hipLaunchKernelGGL(warm_rev_kernel, dim3(N, b.Hv), dim3(256), 0, stream, b.rec, b.Hv, pp.counts,
                       pp.table, pp.seg_chunk0, pp.seq_off, pp.seq_nseg, (int)L.plan.seg_cap, rw, srw);
    if (int rc = gdn::check_launch("gdn_chunk_bwd(replay table)")) return rc;
    b.rev_warm = rw;
    b.seq_rev_warm = srw;
  }
  b.seg_sum = L.plan.split ? reinterpret_cast<float*>(ws + L.plan.off_state) : nullptr;
  b.seg_in = L.plan.split ? reinterpret_cast<float*>(ws + L.plan.off_init) : nullptr;
  const dim3 sgrid((unsigned)L.plan.seg_cap, b.Hv);
  if (L.plan.split) {
    hipLaunchKernelGGL((dstate_kernel<E, DK, DV, true>), sgrid, dim3(DsCfg<E, DK, DV, true>::NT), 0,
                       stream, b);
    if (int rc = gdn::check_launch("gdn_chunk_bwd(dS summaries)")) return rc;
    hipLaunchKernelGGL((seg_scan_kernel<DK, DV, true>), dim3(N, b.Hv, DV / 16), dim3(DK * 2), 0,
                       stream, b.seg_sum, b.seg_in, b.dht, pp.seq_off, pp.seq_nseg, b.Hv,
                       b.seq_rev_warm);
    if (int rc = gdn::check_launch("gdn_chunk_bwd(dS scan)")) return rc;
  }
  if constexpr (std::is_same<E, bf16>::value && DK == DV && (DV == 128 || DV == 64)) {
    // bfloat16 keeps records: the loader / consumer final pass
    static_assert(uses_prep<E, DK, DV, kStates>(), "the final pass reads the prep's records");
    hipLaunchKernelGGL((dsr_kernel<DK, DV>), sgrid, dim3(DsrCfg<DK, DV>::NT), 0, stream, b);
  } else {
    hipLaunchKernelGGL((dstate_kernel<E, DK, DV, false>), sgrid, dim3(DsCfg<E, DK, DV, false>::NT), 0,
                       stream, b);
  }
  if (int rc = gdn::check_launch("gdn_chunk_bwd(dstate)")) return rc;
  if (b.dh0) {  // empty sequences: dh0 = dht (or zero)
    hipLaunchKernelGGL(empty_seq_state_kernel, dim3(N, b.Hv), dim3(256), 0, stream, b.cu, b.dht,
                       b.dh0, b.Hv, DK * DV);
    if (int rc = gdn::check_launch("gdn_chunk_bwd(empty sequences)")) return rc;
  }
  hipLaunchKernelGGL((grad_kernel<E, DK, DV>), dim3((unsigned)L.plan.chunk_cap, b.Hv), dim3(CF::NT),
                     0, stream, b);
  if (int rc = gdn::check_launch("gdn_chunk_bwd(grad)")) return rc;
  if (b.Hv == b.Hk) return GDN_OK;  // the gradient kernel wrote dq and dk itself
  const int64_t units = T * b.Hk;
  constexpr int64_t kUnitsPerBlock = 4 * (64 / (DK / 4));  // four waves
  hipLaunchKernelGGL((finalize_qk_kernel<E, DK>),
                     dim3((unsigned)((units + kUnitsPerBlock - 1) / kUnitsPerBlock)), dim3(256), 0,
                     stream, b, units);
  return gdn::check_launch("gdn_chunk_bwd(finalize)");
}

// dh0 = dht (or 0) for every sequence when there are no tokens at all
__global__ __launch_bounds__(256) void copy_or_zero_kernel(const float* __restrict__ src,
                                                           float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

}  // namespace

extern "C" size_t gdn_chunk_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv,
                                           int32_t dk, int32_t dv, gdn_dtype dt, int bwd) {
  (void)Hk;
  if (T < 0 || N < 0 || Hv < 1 || dk < 1 || dv < 1) return 0;
  if (!bwd) return gdn::chunk_fwd_workspace(T, N, Hv, dk, dv, dt);
  return bwd_layout(T, N, Hv, dk, dv, dt).end;
}

namespace {

int chunk_bwd(const char* fn, const void* q, const void* k, int64_t ld_qk, const void* v,
              int64_t ld_v, const float* g, const float* beta, const float* h0,
              const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk, int32_t Hv, int32_t dk,
              int32_t dv, float scale, int use_qk_l2norm, const void* d_o, const float* dht,
              void* dq, void* dk_, int64_t ld_dqk, void* dv_, int64_t ld_dv, float* dg,
              float* dbeta, float* dh0, const void* saved, size_t saved_bytes, bool use_saved,
              void* ws, size_t ws_bytes, gdn_dtype dt, hipStream_t stream) {
  int rc = gdn::validate_chunk(fn, q, k, ld_qk, v, ld_v, g, beta, cu_seqlens, N, T, Hk, Hv, dk, dv,
                               dt);
  if (rc != GDN_OK) return rc;
  const bool have = (dt == GDN_BF16 && dk == dv && (dk == 128 || dk == 64)) ||
                    (dt == GDN_F32 && dk == dv && (dk == 32 || dk == 64));
  if (!have)
    return gdn::fail(GDN_EUNSUPPORTED,
                     "%s: needs dk == dv (128 or 64 for bfloat16, 32 or 64 for float32)", fn);
  if (T > 0 && (!d_o || !dq || !dk_ || !dv_ || !dg || !dbeta))
    return gdn::fail(GDN_EINVAL, "%s: null gradient pointer", fn);
  if (ld_dqk < (int64_t)Hk * dk || ld_dv < (int64_t)Hv * dv)
    return gdn::fail(GDN_EINVAL, "%s: gradient row strides smaller than the head blocks", fn);
  {
    // a chunk's 64 rows of dq, dk, dv and of the fp32 partial rows are
    // addressed with 32-bit byte offsets
    const int64_t lim = (int64_t)1 << 32, es = dt == GDN_BF16 ? 2 : 4;
    if (64 * ld_dqk * es >= lim || 64 * ld_dv * es >= lim || 64 * (int64_t)Hv * 2 * dk * 4 >= lim)
      return gdn::fail(GDN_EINVAL, "%s: 64 rows of dq, dk or dv must span less than 4 GiB", fn);
  }
  const BwdLayout L = bwd_layout(T, N, Hv, dk, dv, dt);
  if (!ws || ws_bytes < L.end || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return gdn::fail(GDN_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned", fn, L.end);
  if (use_saved) {
    const size_t need = gdn::chunk_saved_layout(T, N, Hv, dk, dv, dt).end;
    if (!saved || saved_bytes < need || (reinterpret_cast<uintptr_t>(saved) & 255u))
      return gdn::fail(GDN_EINVAL, "%s: saved buffer needs %zu bytes, 256-byte aligned", fn, need);
  }
  const char* sv = use_saved ? static_cast<const char*>(saved) : nullptr;
  if (T == 0 || N == 0) {
    if (dh0 && N > 0) {
      const int64_t n = (int64_t)N * Hv * dk * dv;
      hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                         dht, dh0, n);
      return gdn::check_launch("gdn_chunk_bwd(empty)");
    }
    return GDN_OK;
  }
  BwdArgs b{};
  b.q = q;
  b.k = k;
  b.ld_qk = ld_qk;
  b.v = v;
  b.ld_v = ld_v;
  b.g = g;
  b.beta = beta;
  b.Hk = Hk;
  b.Hv = Hv;
  b.scale = scale;
  b.use_l2norm = use_qk_l2norm ? 1 : 0;
  b.d_o = d_o;
  b.dht = dht;
  b.dq = dq;
  b.dk = dk_;
  b.ld_dqk = ld_dqk;
  b.dv = dv_;
  b.ld_dv = ld_dv;
  b.dg = dg;
  b.dbeta = dbeta;
  b.dh0 = dh0;
  b.cu = cu_seqlens;
  b.T = T;
  LoopArgs la{};
  la.q = q;
  la.k = k;
  la.ld_qk = ld_qk;
  la.v = v;
  la.ld_v = ld_v;
  la.g = g;
  la.beta = beta;
  la.h0 = h0;
  la.Hk = Hk;
  la.Hv = Hv;
  la.scale = scale;
  la.use_l2norm = b.use_l2norm;
  if (dt == GDN_BF16) {
    if (dk == 128) return launch_bwd<bf16, 128, 128>(b, la, N, T, L, (char*)ws, sv, stream);
    return launch_bwd<bf16, 64, 64>(b, la, N, T, L, (char*)ws, sv, stream);
  }
  if (dk == 32) return launch_bwd<float, 32, 32>(b, la, N, T, L, (char*)ws, sv, stream);
  return launch_bwd<float, 64, 64>(b, la, N, T, L, (char*)ws, sv, stream);
}

}  // namespace

extern "C" int gdn_chunk_bwd(const void* q, const void* k, int64_t ld_qk, const void* v,
                             int64_t ld_v, const float* g, const float* beta, const float* h0,
                             const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                             int32_t Hv, int32_t dk, int32_t dv, float scale, int use_qk_l2norm,
                             const void* d_o, const float* dht, void* dq, void* dk_,
                             int64_t ld_dqk, void* dv_, int64_t ld_dv, float* dg, float* dbeta,
                             float* dh0, void* ws, size_t ws_bytes, gdn_dtype dt,
                             hipStream_t stream) {
  return chunk_bwd("gdn_chunk_bwd", q, k, ld_qk, v, ld_v, g, beta, h0, cu_seqlens, N, T, Hk, Hv, dk,
                   dv, scale, use_qk_l2norm, d_o, dht, dq, dk_, ld_dqk, dv_, ld_dv, dg, dbeta, dh0,
                   nullptr, 0, false, ws, ws_bytes, dt, stream);
}

extern "C" int gdn_chunk_bwd_saved(const void* q, const void* k, int64_t ld_qk, const void* v,
                                   int64_t ld_v, const float* g, const float* beta,
                                   const float* h0, const int32_t* cu_seqlens, int32_t N,
                                   int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                                   float scale, int use_qk_l2norm, const void* d_o,
                                   const float* dht, void* dq, void* dk_, int64_t ld_dqk,
                                   void* dv_, int64_t ld_dv, float* dg, float* dbeta, float* dh0,
                                   const void* saved, size_t saved_bytes, void* ws,
                                   size_t ws_bytes, gdn_dtype dt, hipStream_t stream) {
  return chunk_bwd("gdn_chunk_bwd_saved", q, k, ld_qk, v, ld_v, g, beta, h0, cu_seqlens, N, T, Hk,
                   Hv, dk, dv, scale, use_qk_l2norm, d_o, dht, dq, dk_, ld_dqk, dv_, ld_dv, dg,
                   dbeta, dh0, saved, saved_bytes, true, ws, ws_bytes, dt, stream);
}
