// chunk_prep.h -- the state-independent part of every chunk, for all chunks
// at once (hyper-parallel "linear_attention_context_parallel.py",
// _prepare_gdn_chunks_for_summary: the prepared chunks that the state pass
// then consumes).
//
// For one chunk of 64 tokens and one value head, with G the in-chunk cumsum
// of g, Gamma_rc = e^{G_r - G_c}, rk the l2norm factors of k and
// L = strict-lower(kh kh^T o Gamma), the chunk's corrected values solve
// (I + diag(beta) L) x = diag(beta)(v - fk o (k S)), fk = e^G rk.  With the
// lower-triangular
//   T = (I + diag(beta) L)^-1 diag(beta)
// that is x = T (v - fk o (k S)), so the state passes need, besides k and v,
// only T and the row factors fk, fd = rk e^{G_C - G} (S <- e^{G_C} S +
// k^T (fd o x)) and eC = e^{G_C}.  The output pass forms the decayed q k^T
// (P) and fo = e^G rq itself from its q rows, G and rk.
//
// T is formed blockwise over 16-row blocks: D_i = (I + diag(beta_i) L_ii)^-1
// (a nilpotent series), A_i = D_i diag(beta_i), E_im = A_i L_im, and then
// T_ii = A_i, T_im = -sum_{m <= j < i} E_ij T_jm: column block m of T only
// involves column block m, so each wave solves one.
//
// One workgroup computes the raw product k k^T of a chunk once per q/k head
// and serves every value head of that head (GQA).  The record of a (chunk,
// value head) stores T as MFMA A fragments in lane order, so the state pass
// copies it into LDS and reads each lane's fragment with one load.
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_common.h"
#include "chunk_plan.h"
#include "gating.h"
#include "gdn_internal.h"

namespace gdn_chunk {

// Record of one (chunk, value head), bytes:
//   [kRecT, +6 KiB)  T as six 16x16x32 A fragments (16 B a lane): row block
//                    mt, contraction half s, for (mt, s) in p_frag order
//   [kRecF, kRecG)   fd[64], fk[64], eC, lb (fp32): lb bounds the log of the
//                    norm of the chunk's state transition (G_C when every
//                    write strength is in [0, 1] and k is l2-normalised, each
//                    token's map then being e^g times a contraction; else
//                    +inf: no bound)
//   [kRecG, kRecEnd) G[64], rk[64] (fp32; read by the output pass only)
constexpr int kRecT = 0;
constexpr int kRecF = 6 * 1024;
constexpr int kRecG = kRecF + 2 * 256 + 16;
constexpr int kRecEnd = kRecG + 2 * 256;
constexpr int kRecBytes = 7424;  // record stride, a multiple of 256 bytes
static_assert(kRecEnd <= kRecBytes && kRecG % 16 == 0 && kRecEnd % 16 == 0, "record layout");

// Fragments of a 64 x 64 lower-triangular operator that are not entirely
// above the diagonal: (row block mt, contraction half s) -> index.
__host__ __device__ constexpr int p_frag(int mt, int s) { return mt == 0 ? 0 : mt == 1 ? 1 : 2 * mt - 2 + s; }

namespace {

constexpr int kPrepScLd = 20;    // fp32 16 x 16 scratch rows (16 + 4)

// fp32 16 x 16 tiles of the staging area, per wave w from prep_tile0(w):
// wave 0: L_00 and a work tile; wave w > 0: L_ww and the work tile of its
// inversion, which then hold A_w and E_w0, followed by E_w1 .. E_w,w-1.  The
// first tile of a wave is read by that wave only; it finally turns T's tiles
// into fragment lane order.
__host__ __device__ constexpr int prep_tile0(int w) { return w == 0 ? 0 : w * (w + 1) / 2 + 1; }
constexpr int kPrepTiles = 11;

// The raw rows are dead once the products are formed, so the per-head staging
// shares their space (19.7 KB a workgroup; seven a CU, held by registers).
template <int DK>
struct PrepSmem {
  static constexpr int LDK = DK + 8;
  struct Stage {
    alignas(16) float sc[kPrepTiles][16 * kPrepScLd];
  };
  union {
    alignas(16) bf16 k[64 * LDK];  // raw rows, dead once k k^T is formed
    Stage s;
  } u;
  alignas(16) float rk[64];
  alignas(16) float wv[4][2][64];  // per wave: G, beta
};

struct PrepArgs {
  const void* k;
  int64_t ld_qk;
  gdn_gate::Gates gates;  // given g, beta, or the projections they are formed from
  int Hk, Hv;
  int use_l2norm;
  const int4* chunk_tab;
  const int32_t* counts;
  char* rec;
};

// (I + N)^-1 for N = diag(bb) L, L strictly lower 16 x 16 (Lt: fp32, rows of
// kPrepScLd), NC: N in C layout; sc: work tile.  N^16 = 0, so the inverse is
// (I - N)(I + N^2)(I + N^4)(I + N^8): six fp32 products.  Returns C layout.
GDN_DEV floatx4 prep_invert16(const float* Lt, const float* bb, const floatx4& NC, float* sc, int lane) {
  typedef Tile16<float> F;
  const int g4 = lane >> 4, ln = lane & 15;
  const floatx4 NA = F::load_f32(Lt, kPrepScLd, 0, 0, bb[ln], lane);
  floatx4 N2 = zero4();
  F::mma(N2, NA, NC);
#pragma unroll
  for (int j = 0; j < 4; j++) sc[(4 * g4 + j) * kPrepScLd + ln] = N2[j];
  wave_lds_sync();
  const floatx4 N2A = F::load(sc, kPrepScLd, 0, 0, lane);
  floatx4 N4 = zero4();
  F::mma(N4, N2A, N2);
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 4; j++) sc[(4 * g4 + j) * kPrepScLd + ln] = N4[j];
  wave_lds_sync();
  const floatx4 N4A = F::load(sc, kPrepScLd, 0, 0, lane);
  floatx4 N8 = zero4();
  F::mma(N8, N4A, N4);
  floatx4 R1 = N4 + N8;
#pragma unroll
  for (int j = 0; j < 4; j++) R1[j] += (4 * g4 + j == ln) ? 1.f : 0.f;
  F::mma(R1, N4A, N8);
  floatx4 R2 = R1;
  F::mma(R2, N2A, R1);
  floatx4 t = zero4();
  F::mma(t, NA, R2);
  return R2 - t;
}

// Column block W of T: T_WW = A_W (Ai), T_iW = -sum_{W <= j < i} E_ij T_jW
// for i > W (E_ij from wave i's tiles).  Block W is half W % 2 (bytes
// 8(W % 2) .. + 7 of each lane's 16) of the fragments of contraction slab
// W / 2, where lane l holds row l%16 and columns 4(l/16) .. + 3 of the block:
// each tile goes from C layout through this wave's own tile Lt (A_W is no
// longer read) and its half is stored straight to the record.
template <int W, class SM>
GDN_DEV void prep_column(SM& sm, const floatx4& Ai, float* Lt, char* rec, int lane) {
  typedef Tile16<float> F;
  const int g4 = lane >> 4, ln = lane & 15;
  floatx4 Tc[4];
  Tc[W] = Ai;
#pragma unroll
  for (int i = W + 1; i < 4; i++) {
    floatx4 acc = zero4();
#pragma unroll
    for (int j = W; j < i; j++)
      F::mma(acc, F::load(sm.u.s.sc[prep_tile0(i) + 1 + j], kPrepScLd, 0, 0, lane), Tc[j]);
    Tc[i] = -acc;
  }
  char* tdst = rec + kRecT + 8 * (W & 1) + 16 * lane;
  if constexpr (W & 1)  // the zero block above the diagonal in row block W - 1
    *reinterpret_cast<bf16x4*>(tdst + p_frag(W - 1, W >> 1) * 1024) = bf16x4{};
#pragma unroll
  for (int i = W; i < 4; i++) {
#pragma unroll
    for (int jj = 0; jj < 4; jj++) Lt[(4 * g4 + jj) * kPrepScLd + ln] = Tc[i][jj];
    wave_lds_sync();
    const floatx4 tv = *reinterpret_cast<const floatx4*>(Lt + ln * kPrepScLd + 4 * g4);
    bf16x4 b;
#pragma unroll
    for (int e = 0; e < 4; e++) b[e] = (bf16)tv[e];
    *reinterpret_cast<bf16x4*>(tdst + p_frag(i, W >> 1) * 1024) = b;
    wave_lds_sync();  // read before the next tile overwrites
  }
}

// One (chunk, q/k head) per workgroup of four waves.  Wave w owns the L
// blocks of row block w (L_ww, L_wm for m < w: the inversion and E_wm stay in
// the wave) and column block w of T.
template <int DK>
#ifndef GDN_PREP_WAVES
#define GDN_PREP_WAVES 6
#endif
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GDN_PREP_WAVES))) void chunk_prep_kernel(PrepArgs a) {
  typedef Mfma<bf16> M;
  typedef M::frag Fr;
  typedef Tile16<float> F;
  typedef PrepSmem<DK> SM;
  constexpr int LDK = SM::LDK;
  constexpr int NSK = DK / 32;
  __shared__ SM sm;

  // Workgroup order: the q/k heads of one chunk take ids 8 apart, so they run
  // together on one XCD (ids go round-robin over the 8 XCDs) and read the
  // chunk's lines of g and beta (all heads of a token share a line) through
  // its L2 once.
  const int id = blockIdx.x;
  const int qa = (id >> 3) % a.Hk, chunk = (id / (8 * a.Hk)) * 8 + (id & 7);
  if (chunk >= a.counts[1]) return;
  const int4 ce = a.chunk_tab[chunk];
  const int64_t tc = ce.x, te = ce.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, ln = lane & 15;
  const int GR = a.Hv / a.Hk;

  // gates of the 64 tokens, one per lane (zero past the end), for the first
  // value head: issued first, so they arrive with the rows; the next value
  // head's are loaded one head ahead
  const int64_t tg = tc + lane;
  float gn = 0.f, bn = 0.f;
  if (tg < te) gdn_gate::load_gates<bf16>(a.gates, tg, qa * GR, a.Hv, gn, bn);

  // raw k rows (zero past the sequence end) and their l2norm factors; every
  // load reads a valid row (past the end the chunk's first, zeroed after) and
  // all are issued before the first store, so they are in flight together
  {
    typedef bf16x8 V;
    constexpr int QPR = DK / 8, KP = 64 * QPR / 256;
    const bf16* kp = (const bf16*)a.k + (int64_t)qa * DK;
    V kr[KP];
#pragma unroll
    for (int p = 0; p < KP; p++) {
      const int i = tid + 256 * p;
      const int64_t t = tc + i / QPR;
      kr[p] = *reinterpret_cast<const V*>(kp + (t < te ? t : tc) * a.ld_qk + (i % QPR) * 8);
    }
#pragma unroll
    for (int p = 0; p < KP; p++) {
      const int i = tid + 256 * p;
      const int row = i / QPR, vi = i % QPR;
      const V kv = tc + row < te ? kr[p] : zero_vec16<bf16>();
      *reinterpret_cast<V*>(sm.u.k + row * LDK + vi * 8) = kv;
      const float ks = row_group_sum<QPR>(sum_sq(kv));
      if (vi == 0) sm.rk[row] = a.use_l2norm ? __builtin_amdgcn_rsqf(ks + 1e-6f) : 1.f;
    }
  }
  __syncthreads();

  // raw products of this wave's blocks: k_w k_w^T and k_w k_t^T (t < w)
  floatx4 rD = zero4(), rO[3];
#pragma unroll
  for (int t = 0; t < 3; t++) rO[t] = zero4();
#pragma unroll
  for (int s = 0; s < NSK; s++) {
    const Fr ak = M::load(sm.u.k, LDK, 16 * w, 32 * s, lane);
    M::mma(rD, ak, ak);
#pragma unroll
    for (int t = 0; t < 3; t++)
      if (t < w) M::mma(rO[t], ak, M::load(sm.u.k, LDK, 16 * t, 32 * s, lane));
  }
  float rkL[4];
#pragma unroll
  for (int jj = 0; jj < 4; jj++) rkL[jj] = sm.rk[16 * w + 4 * g4 + jj];
  __syncthreads();  // every wave's products are formed: the rows' space is reused
  float* const tiles = sm.u.s.sc[prep_tile0(w)];
  float* Lt = tiles;                   // L_ww, then A_w
  float* wk = tiles + 16 * kPrepScLd;  // work tile, then E_w0
  float* G = sm.wv[w][0];
  float* bt = sm.wv[w][1];

  for (int r = 0; r < GR; r++) {
    const int h = qa * GR + r;
    char* rec = a.rec + ((int64_t)chunk * a.Hv + h) * kRecBytes;
    const float gv = gn, bv = bn;
    if (r + 1 < GR && tg < te) gdn_gate::load_gates<bf16>(a.gates, tg, h + 1, a.Hv, gn, bn);
    const float Gv = wave_incl_scan(gv);  // in-chunk cumsum of g
    const float GC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gv), 63));
    const float egv = __expf(Gv);
    const float fkv = egv * sm.rk[lane];
    G[lane] = Gv;
    bt[lane] = bv;
    if (w == 0) {
      float* F32 = reinterpret_cast<float*>(rec + kRecF);
      F32[lane] = sm.rk[lane] * __expf(GC - Gv);  // fd
      F32[64 + lane] = fkv;                       // fk
      if (lane == 0) F32[128] = __expf(GC);       // eC
      // every valid token's beta in [0, 1] (past the end beta = 0)
      const bool contract = a.use_l2norm && __all(bv >= 0.f && bv <= 1.f);
      if (lane == 0) F32[129] = contract ? GC : __builtin_inff();  // lb
      float* G32 = reinterpret_cast<float*>(rec + kRecG);
      G32[lane] = Gv;
      G32[64 + lane] = sm.rk[lane];
    }
    wave_lds_sync();

    // diagonal L block -> fp32 scratch, then D and A_w = D diag(beta)
    floatx4 NC;
    {
      const int c = 16 * w + ln;
      const float Gc = G[c], fc = sm.rk[c];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) {
        const int row = 16 * w + 4 * g4 + jj;
        const float e = __expf(fminf(G[row] - Gc, 0.f));  // clamped: masked entries stay finite
        const float val = row > c ? rD[jj] * rkL[jj] * fc * e : 0.f;
        Lt[(4 * g4 + jj) * kPrepScLd + ln] = val;
        NC[jj] = bt[row] * val;
      }
    }
    wave_lds_sync();
    const floatx4 D = prep_invert16(Lt, bt + 16 * w, NC, wk, lane);
    floatx4 Ai;
    {
      const float bc = bt[16 * w + ln];
#pragma unroll
      for (int jj = 0; jj < 4; jj++) Ai[jj] = D[jj] * bc;
    }
    // E_wm = A_w L_wm for m < w (A_w as A operand through LDS), kept in fp32
    // for the column solves of the other waves
    if (w > 0) {
      wave_lds_sync();  // the inversion's last reads of its tiles are done
#pragma unroll
      for (int jj = 0; jj < 4; jj++) Lt[(4 * g4 + jj) * kPrepScLd + ln] = Ai[jj];
      wave_lds_sync();
      const floatx4 AA = F::load(Lt, kPrepScLd, 0, 0, lane);
      const float G0 = G[16 * w];
#pragma unroll
      for (int t = 0; t < 3; t++) {
        if (t >= w) break;
        const int c = 16 * t + ln;
        // decay factored as e^{G_r - G_0} e^{G_0 - G_c}, both <= 1
        const float bcol = sm.rk[c] * __expf(G0 - G[c]);
        floatx4 Lm;
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
          const int row = 16 * w + 4 * g4 + jj;
          Lm[jj] = rO[t][jj] * rkL[jj] * __expf(G[row] - G0) * bcol;
        }
        floatx4 E = zero4();
        F::mma(E, AA, Lm);
        float* et = wk + t * (16 * kPrepScLd);
#pragma unroll
        for (int jj = 0; jj < 4; jj++) et[(4 * g4 + jj) * kPrepScLd + ln] = E[jj];
      }
    }
    __syncthreads();  // every E block is in place
    // column block m = w of T (the wave index fixed at compile time, so the
    // products that do not wait on the block above interleave)
    switch (w) {
      case 0: prep_column<0>(sm, Ai, Lt, rec, lane); break;
      case 1: prep_column<1>(sm, Ai, Lt, rec, lane); break;
      case 2: prep_column<2>(sm, Ai, Lt, rec, lane); break;
      default: prep_column<3>(sm, Ai, Lt, rec, lane); break;
    }
    __syncthreads();  // staging is rewritten for the next value head
  }
}

template <int DK>
int launch_prep(const PrepArgs& a, int64_t chunk_cap, hipStream_t stream) {
  const int64_t n = (chunk_cap + 7) / 8 * 8 * a.Hk;
  hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3((unsigned)n), dim3(256), 0, stream, a);
  return gdn::check_launch("chunk prep");
}

}  // namespace
}  // namespace gdn_chunk
