// chunk_common.h -- per-chunk machinery of the chunked gated delta rule,
// shared by the forward and backward kernels.
//
// hyper-parallel "linear_attention_context_parallel.py",
// _prepare_gdn_chunks_for_summary, evaluated for one (chunk, value head) in
// one workgroup with every intermediate on chip:
//   qh, kh    l2-normalised q (times scale) and k            (_l2norm_torch)
//   G         in-chunk cumulative sum of g
//   L         strict-lower( diag(beta) kh kh^T o exp(G_i - G_j) ); the LDS
//             copy holds it without diag(beta), which the solve applies
//   P         lower-incl( qh kh^T o exp(G_i - G_j) )      (the output's attn)
//   T         (I + L)^-1, unit lower triangular
//   u         T diag(beta) v                              (chunk_value)
//   w         T diag(beta exp(G)) kh                      (k_cumdecay)
// The page forms T by a 63-step row recurrence; here the four 16x16
// diagonal blocks are inverted by column-oriented forward substitution (one
// wave, one lane per column, while the other waves form P) and the
// off-diagonal blocks follow from T_ij = -T_ii sum_{m=j}^{i-1} L_im T_mj on
// fp32 MFMA, one block distance at a time.  Products with token-sized
// contraction use bf16 MFMA with fp32 accumulation (fp32 MFMA for float32
// activations); see gdn_common.h for the fragment convention.
//
// LDS (one workgroup = one chunk of one head at a time), rows padded by 16
// bytes: q, k [64][DK], v [64][DV], w [64][DK] and p [64][64] in the operand
// type; L and Tm [64][68] fp32; G, beta, beta*exp(G), exp(G) [64] fp32.  Operands
// whose contraction index is the token (k in w and in the state update, v
// in u) are read down columns of the row-major copies.
#pragma once

#include "gdn_common.h"

namespace gdn_chunk {

constexpr int BT = 64;  // chunk length

template <typename O, int DK, int DV, bool HAS_Q>
struct Smem {
  static constexpr int PAD = 16 / (int)sizeof(O);
  static constexpr int LDK = DK + PAD;  // row-major [BT][DK]
  static constexpr int LDV = DV + PAD;  // row-major [BT][DV]
  static constexpr int LDT = BT + PAD;  // [BT][BT] operand arrays
  static constexpr int LDF = BT + 4;    // fp32 [BT][BT]
  alignas(16) O q[HAS_Q ? BT * LDK : 8];
  alignas(16) O k[BT * LDK];
  alignas(16) O v[BT * LDV];
  alignas(16) O w[BT * LDK];
  alignas(16) O p[HAS_Q ? BT * LDT : 8];
  alignas(16) float L[BT * LDF];
  alignas(16) float Tm[BT * LDF];
  alignas(16) float G[BT];
  alignas(16) float beta[BT];
  alignas(16) float bg[BT];  // beta * exp(G)
  alignas(16) float eg[BT];  // exp(G)
  alignas(16) float rnq[BT];  // l2norm factors of the raw q, k rows (1 without)
  alignas(16) float rnk[BT];
};

// Global -> register prefetch of one chunk (q, k rows of q/k head `qa`, v
// rows of value head `h` unless HAS_V is false, g and beta of head h).
template <typename E, int DK, int DV, int NT, bool HAS_Q, bool HAS_V = true>
struct Prefetch {
  typedef typename Vec16<E>::type V16;
  static constexpr int VE = Vec16<E>::N;
  static constexpr int QPR = DK / VE;  // 16-byte vectors per q/k row
  static constexpr int VPR = DV / VE;
  static constexpr int QV = BT * QPR;
  static constexpr int VV = BT * VPR;
  static constexpr int PQ = (QV + NT - 1) / NT;
  static constexpr int PV = HAS_V ? (VV + NT - 1) / NT : 0;
  V16 q[HAS_Q ? PQ : 1];
  V16 k[PQ];
  V16 v[PV > 0 ? PV : 1];
  float g, beta;

  GDN_DEV void load(const E* __restrict__ qp, const E* __restrict__ kp, int64_t ld_qk,
                    const E* __restrict__ vp, int64_t ld_v, const float* __restrict__ gp,
                    const float* __restrict__ bp, int Hv, int64_t tc, int64_t te, int tid) {
    // Every load reads a valid row (past the sequence end or the tile: the
    // chunk's first row, which always holds a token) and the unused ones are
    // zeroed after, so no load sits behind a branch and all are in flight at
    // once.
#pragma unroll
    for (int p = 0; p < PQ; p++) {
      const int i = tid + NT * p;
      const int64_t t = tc + i / QPR;
      const bool ok = (i < QV) && (t < te);
      const int64_t off = (ok ? t : tc) * ld_qk + (ok ? i % QPR : 0) * VE;
      if constexpr (HAS_Q) q[p] = *reinterpret_cast<const V16*>(qp + off);
      k[p] = *reinterpret_cast<const V16*>(kp + off);
    }
#pragma unroll
    for (int p = 0; p < PV; p++) {
      const int i = tid + NT * p;
      const int64_t t = tc + i / VPR;
      const bool ok = (i < VV) && (t < te);
      v[p] = *reinterpret_cast<const V16*>(vp + (ok ? t : tc) * ld_v + (ok ? i % VPR : 0) * VE);
    }
#pragma unroll
    for (int p = 0; p < PQ; p++) {
      const int i = tid + NT * p;
      if (!((i < QV) && (tc + i / QPR < te))) {
        if constexpr (HAS_Q) q[p] = zero_vec16<E>();
        k[p] = zero_vec16<E>();
      }
    }
#pragma unroll
    for (int p = 0; p < PV; p++) {
      const int i = tid + NT * p;
      if (!((i < VV) && (tc + i / VPR < te))) v[p] = zero_vec16<E>();
    }
    g = 0.f;
    beta = 0.f;
    if (tid < BT && tc + tid < te) {
      g = gp[(tc + tid) * Hv];
      beta = bp[(tc + tid) * Hv];
    }
  }
};

// Register prefetch -> LDS: l2norm (and q scale), row-major copies (16-byte
// stores), in-chunk cumsum of g.  Rows past the sequence end are zero, which
// leaves the state untouched (the page's zero padding).
template <typename E, typename O, int DK, int DV, int NT, bool HAS_Q, class SM>
GDN_DEV void stage(SM& sm, const Prefetch<E, DK, DV, NT, HAS_Q>& pf, float scale, int use_l2norm,
                   int tid) {
  typedef Prefetch<E, DK, DV, NT, HAS_Q> PF;
  typedef typename Vec16<O>::type OV;
  constexpr int VE = PF::VE;
  static_assert(sizeof(E) == sizeof(O), "activation and operand types must match");
#pragma unroll
  for (int p = 0; p < PF::PQ; p++) {
    const int i = tid + NT * p;
    const int row = i / PF::QPR, vi = i % PF::QPR;
    float kf[VE], qf[VE];
    float kss = 0.f, qss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; e++) {
      kf[e] = to_f(pf.k[p][e]);
      kss += kf[e] * kf[e];
      if constexpr (HAS_Q) {
        qf[e] = to_f(pf.q[p][e]);
        qss += qf[e] * qf[e];
      }
    }
    kss = group_sum<PF::QPR>(kss);
    const float kr = use_l2norm ? 1.f / sqrtf(kss + 1e-6f) : 1.f;
    float qr = scale;
    if constexpr (HAS_Q) {
      qss = group_sum<PF::QPR>(qss);
      if (use_l2norm) qr = scale / sqrtf(qss + 1e-6f);
    }
    if (i < PF::QV && vi == 0) {
      sm.rnk[row] = kr;
      if constexpr (HAS_Q) sm.rnq[row] = use_l2norm ? 1.f / sqrtf(qss + 1e-6f) : 1.f;
    }
    if (i < PF::QV) {
      OV kv, qv;
#pragma unroll
      for (int e = 0; e < VE; e++) {
        kv[e] = from_f<O>(kf[e] * kr);
        if constexpr (HAS_Q) qv[e] = from_f<O>(qf[e] * qr);
      }
      *reinterpret_cast<OV*>(sm.k + row * SM::LDK + vi * VE) = kv;
      if constexpr (HAS_Q) *reinterpret_cast<OV*>(sm.q + row * SM::LDK + vi * VE) = qv;
    }
  }
#pragma unroll
  for (int p = 0; p < PF::PV; p++) {
    const int i = tid + NT * p;
    const int row = i / PF::VPR, vi = i % PF::VPR;
    if (i < PF::VV) *reinterpret_cast<OV*>(sm.v + row * SM::LDV + vi * VE) = pf.v[p];
  }
  if (tid < BT) {  // wave 0: inclusive scan of g over the 64 rows (DPP, as the prep's)
    const float G = wave_incl_scan(pf.g);
    const float eG = __expf(G);
    sm.G[tid] = G;
    sm.beta[tid] = pf.beta;
    sm.bg[tid] = pf.beta * eG;
    sm.eg[tid] = eG;
  }
}

// One lower 16x16 tile (i, j), j <= i, of kh kh^T (-> strict-lower L
// without beta, fp32) or qh kh^T (-> P, operand type), with the decay
// exp(G_row - G_col) applied.
template <typename O, int DK, class SM>
GDN_DEV void gram_tile(SM& sm, bool isq, int i, int j, int lane) {
  typedef Mfma<O> M;
  floatx4 acc = zero4();
  const O* A = isq ? sm.q : sm.k;
#pragma unroll
  for (int s = 0; s < DK / M::KSTEP; s++)
    M::mma(acc, M::load(A, SM::LDK, 16 * i, s * M::KSTEP, lane),
           M::load(sm.k, SM::LDK, 16 * j, s * M::KSTEP, lane));
  const int col = 16 * j + (lane & 15);
  const int rb = 16 * i + 4 * (lane >> 4);
  const float Gc = sm.G[col];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) {
    const int row = rb + jj;
    const float dec = row >= col ? __expf(sm.G[row] - Gc) : 0.f;
    if (!isq) {
      sm.L[row * SM::LDF + col] = row > col ? acc[jj] * dec : 0.f;
    } else {
      sm.p[row * SM::LDT + col] = from_f<O>(acc[jj] * dec);
    }
  }
}

GDN_DEV void lower_tile_ij(int idx, int& i, int& j) {
  i = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
  j = idx - i * (i + 1) / 2;
}

// L tiles (all waves).
template <typename O, int DK, int NW, class SM>
GDN_DEV void gram_kk(SM& sm, int wave, int lane) {
  for (int t = wave; t < 10; t += NW) {
    int i, j;
    lower_tile_ij(t, i, j);
    gram_tile<O, DK>(sm, false, i, j, lane);
  }
}

// Zero the strictly-upper 16x16 tiles of L, Tm and P (never written later).
template <typename O, bool HAS_Q, int NT, class SM>
GDN_DEV void zero_upper(SM& sm, int tid) {
  for (int e = tid; e < BT * BT; e += NT) {
    const int r = e / BT, c = e % BT;
    if ((c >> 4) > (r >> 4)) {
      sm.L[r * SM::LDF + c] = 0.f;
      sm.Tm[r * SM::LDF + c] = 0.f;
      if constexpr (HAS_Q) sm.p[r * SM::LDT + c] = from_f<O>(0.f);
    }
  }
}

// T = (I + L)^-1 into sm.Tm; with HAS_Q the P tiles are formed by the waves
// that do not invert.  Needs a barrier before (L complete); ends with one.
template <typename O, int DK, int NW, bool HAS_Q, class SM>
GDN_DEV void solve(SM& sm, int wave, int lane) {
  constexpr int LDF = SM::LDF;
  if (wave == 0) {
    // diagonal blocks: lane (b, j) computes column j of (I + L_bb)^-1 by
    // column-oriented substitution (x_m final after step m)
    const int b = lane >> 4, j = lane & 15;
    const float* Lb = sm.L + (16 * b) * LDF + 16 * b;
    const float* bb = sm.beta + 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; i++) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; m++) {
#pragma unroll
      for (int i = m + 1; i < 16; i++) x[i] -= bb[i] * Lb[i * LDF + m] * x[m];
    }
    float* Tb = sm.Tm + (16 * b) * LDF + 16 * b;
#pragma unroll
    for (int i = 0; i < 16; i++) Tb[i * LDF + j] = x[i];
  }
  if constexpr (HAS_Q) {
    // P tiles on the other waves (or wave 0 alone when there is one wave)
    constexpr int WP = NW > 1 ? NW - 1 : 1;
    const int wp = NW > 1 ? wave - 1 : 0;
    if (NW == 1 || wave > 0)
      for (int t = wp; t < 10; t += WP) {
        int i, j;
        lower_tile_ij(t, i, j);
        gram_tile<O, DK>(sm, true, i, j, lane);
      }
  }
  __syncthreads();
  // off-diagonal blocks, by distance d = i - j
  for (int d = 1; d < 4; d++) {
    for (int blk = wave; blk < 4 - d; blk += NW) {
      const int j = blk, i = blk + d;
      floatx4 r = zero4();
      const float brow = sm.beta[16 * i + (lane & 15)];  // L = diag(beta) (kh kh^T o Gamma)
      for (int m = j; m < i; m++) {
        // A = L_im (rows 16i, cols 16m); B[k][n] = Tm[16m+k][16j+n]
        Mfma<float>::mma(r, Mfma<float>::load(sm.L, LDF, 16 * i, 16 * m, lane) * brow,
                         Mfma<float>::load_col(sm.Tm + 16 * m * LDF, LDF, 16 * j, 0, lane));
      }
      // T_ij = -T_ii r  (r is already in B layout: its rows are k)
      floatx4 o = zero4();
      Mfma<float>::mma(o, Mfma<float>::load(sm.Tm, LDF, 16 * i, 16 * i, lane), r);
      const int rb = 16 * i + 4 * (lane >> 4), c = 16 * j + (lane & 15);
#pragma unroll
      for (int jj = 0; jj < 4; jj++) sm.Tm[(rb + jj) * LDF + c] = -o[jj];
    }
    __syncthreads();
  }
}

// u tiles for 16 NN value columns [vc0, vc0 + 16 NN) into registers (C
// layout, u[mt][nt]: token rows 16mt.., value cols vc0+16nt..).
template <typename O, int NN, class SM>
GDN_DEV void compute_u(const SM& sm, int vc0, int lane, floatx4 (&u)[4][NN]) {
  typedef Mfma<O> M;
  constexpr int NS = BT / M::KSTEP;
  typename M::frag b[NN][NS];
#pragma unroll
  for (int nt = 0; nt < NN; nt++)
#pragma unroll
    for (int s = 0; s < NS; s++) b[nt][s] = M::load_col(sm.v, SM::LDV, vc0 + 16 * nt, s * M::KSTEP, lane);
#pragma unroll
  for (int mt = 0; mt < 4; mt++) {
    floatx4 acc[NN];
#pragma unroll
    for (int nt = 0; nt < NN; nt++) acc[nt] = zero4();
#pragma unroll
    for (int s = 0; s < NS; s++) {
      const typename M::frag a = M::load_scaled(sm.Tm, SM::LDF, 16 * mt, s * M::KSTEP, sm.beta, lane);
#pragma unroll
      for (int nt = 0; nt < NN; nt++) M::mma(acc[nt], a, b[nt][s]);
    }
#pragma unroll
    for (int nt = 0; nt < NN; nt++) u[mt][nt] = acc[nt];
  }
}

// w = T diag(beta exp(G)) kh into sm.w (operand type), tiles spread over waves.
template <typename O, int DK, int NW, class SM>
GDN_DEV void compute_w(SM& sm, int wave, int lane) {
  typedef Mfma<O> M;
  constexpr int NS = BT / M::KSTEP;
  constexpr int NTILE = 4 * (DK / 16);
  // with NW a multiple of 4 every tile of a wave lies in row block wave % 4:
  // its scaled T fragments are formed once
  constexpr bool ONE_ROW = NW % 4 == 0;
  typename M::frag af[NS];
  if constexpr (ONE_ROW) {
#pragma unroll
    for (int s = 0; s < NS; s++) af[s] = M::load_scaled(sm.Tm, SM::LDF, 16 * (wave % 4), s * M::KSTEP, sm.bg, lane);
  }
  for (int tt = wave; tt < NTILE; tt += NW) {
    const int mt = tt % 4, nt = tt / 4;
    floatx4 acc = zero4();
#pragma unroll
    for (int s = 0; s < NS; s++)
      M::mma(acc, ONE_ROW ? af[s] : M::load_scaled(sm.Tm, SM::LDF, 16 * mt, s * M::KSTEP, sm.bg, lane),
             M::load_col(sm.k, SM::LDK, 16 * nt, s * M::KSTEP, lane));
    const int rb = 16 * mt + 4 * (lane >> 4), c = 16 * nt + (lane & 15);
#pragma unroll
    for (int jj = 0; jj < 4; jj++) sm.w[(rb + jj) * SM::LDK + c] = from_f<O>(acc[jj]);
  }
}

// B fragment for contraction step s from accumulator tiles X[kt][nt] whose
// rows are the contraction index.
template <typename O, int NKT, int NN>
GDN_DEV typename Mfma<O>::frag acc_as_b(const floatx4 (&X)[NKT][NN], int s, int nt) {
  if constexpr (Mfma<O>::KSTEP == 32)
    return Mfma<O>::from_acc(X[2 * s][nt], X[2 * s + 1][nt]);
  else
    return Mfma<O>::from_acc(X[s][nt]);
}

}  // namespace gdn_chunk
