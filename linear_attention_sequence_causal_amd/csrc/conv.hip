// conv.hip -- causal depthwise conv1d + SiLU with a carried-in halo, forward
// and reverse mode.
//
// hyper-parallel "linear_attention_context_parallel.py",
// _causal_conv1d_with_cp_halo: per channel c, token t of sequence n,
//   z[t,c] = bias[c] + sum_{j<K} w[c,j] * xh[t-(K-1)+j, c],  y = z*sigmoid(z)
// where xh is x inside the sequence, the last n_halo rows of the halo before
// local sequence 0 (the previous shard's K-1 pre-conv tokens), zero otherwise.
//
// Design (HBM-bound stencil): a thread owns one 16-byte vector of channels
// and a run of R consecutive tokens.  A wave's 64 lanes cover 1 KiB of one
// token row, so every row load and store is fully coalesced.  All rows of
// the run (plus the K-1 rows before it) are loaded up front, so R+K-1
// independent loads are in flight per thread; the K-1 overlap rows are the
// only re-reads and hit L2.  Sequence boundaries only change which taps are
// masked, so the unrolled loop keeps every row in registers.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_common.h"
#include "gdn_internal.h"

namespace {

constexpr int kRunsPerBlock = 4;   // blockDim.y
constexpr int kLanes = 64;         // blockDim.x: channel vectors per block
constexpr int kFwdRows = 8;        // tokens per thread run, forward
constexpr int kBwdRows = 16;       // tokens per thread run, backward
// backward shape: four channels a thread (8-byte rows for bfloat16, which
// leaves registers for three waves a SIMD and four rows in flight ahead of
// the one formed; 16-byte rows, two waves a SIMD and three rows for float32)
template <typename E> struct BwdShape {
  static constexpr int V = 4;
  static constexpr int PD = sizeof(E) == 2 ? 4 : 3;
  static constexpr int WAVES = sizeof(E) == 2 ? 3 : 2;  // a SIMD; also four-wave blocks a CU
};
constexpr int kBwdMaxSplits = 64;  // most token splits of the backward grid (dw partial rows)

// V channels of one row: a packed 16-byte vector when V*sizeof(E) == 16
// (bf16 stays two to a register), else V scalars.
template <typename E, int V, bool VEC = (V * sizeof(E) == 16 || V * sizeof(E) == 8)> struct Row;
template <typename E, int V> struct Row<E, V, true> {
  typedef E VT __attribute__((ext_vector_type(V)));
  VT v;
  GDN_DEV float at(int i) const { return to_f(v[i]); }
};
template <typename E, int V> struct Row<E, V, false> {
  E v[V];
  GDN_DEV float at(int i) const { return to_f(v[i]); }
};

template <typename E, int V>
__device__ __forceinline__ Row<E, V> load_row(const E* p) {
  Row<E, V> r;
  if constexpr (V * sizeof(E) == 16 || V * sizeof(E) == 8) {
    r.v = *reinterpret_cast<const typename Row<E, V>::VT*>(p);
  } else {
#pragma unroll
    for (int i = 0; i < V; i++) r.v[i] = p[i];
  }
  return r;
}

// NT: a non-temporal store (streamed past the caches; the conv's outputs, y
// and dx, are not read again before they would leave them)
template <typename E, int V, bool NT = false>
__device__ __forceinline__ void store_row(E* p, const float* f) {
  if constexpr (V * sizeof(E) == 16 || V * sizeof(E) == 8) {
    typedef typename Row<E, V>::VT VT;
    VT t;
#pragma unroll
    for (int i = 0; i < V; i++) t[i] = from_f<E>(f[i]);
    if constexpr (NT)
      __builtin_nontemporal_store(t, reinterpret_cast<VT*>(p));
    else
      *reinterpret_cast<VT*>(p) = t;
  } else {
#pragma unroll
    for (int i = 0; i < V; i++) p[i] = from_f<E>(f[i]);
  }
}

template <typename E, int V>
__device__ __forceinline__ Row<E, V> zero_row() {
  Row<E, V> r;
  if constexpr (V * sizeof(E) == 16 || V * sizeof(E) == 8) {
    r.v = typename Row<E, V>::VT{};
  } else {
#pragma unroll
    for (int i = 0; i < V; i++) r.v[i] = from_f<E>(0.f);
  }
  return r;
}

// Index n with cu[n] <= t < cu[n+1] (the last such n when sequences are
// empty); requires cu[0] <= t < cu[N].
__device__ __forceinline__ int find_seq(const int32_t* cu, int N, int64_t t) {
  int lo = 0, hi = N;  // invariant: cu[lo] <= t, answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename E, int K, int V>
__global__ __launch_bounds__(kLanes* kRunsPerBlock) void conv_fwd_kernel(
    const E* __restrict__ x, const E* __restrict__ w, const E* __restrict__ bias,
    const E* __restrict__ halo, const int32_t* __restrict__ cu, int N, int64_t T, int C,
    int64_t ldx, int cgroups, const gdn_cp_meta* __restrict__ meta, E* __restrict__ y) {
  constexpr int R = kFwdRows;
  // channel groups vary fastest so that concurrent blocks cover whole rows
  const int64_t b = blockIdx.x;
  const int cg = (int)(b % cgroups);
  const int64_t tile = b / cgroups;
  const int c0 = (cg * kLanes + threadIdx.x) * V;
  const int64_t t0 = (tile * kRunsPerBlock + threadIdx.y) * R;
  if (c0 >= C || t0 >= T) return;
  const int n_halo = (halo && meta) ? meta->n_halo : 0;

  float wv[K][V], bv[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    bv[i] = bias ? to_f(bias[c0 + i]) : 0.f;
#pragma unroll
    for (int j = 0; j < K; j++) wv[j][i] = to_f(w[(c0 + i) * K + j]);
  }
  // rows t0-(K-1) .. t0+R-1 (those inside [0, T)) go out before the sequence
  // search, so the two latencies overlap
  Row<E, V> xr[R + K - 1];
#pragma unroll
  for (int i = 0; i < R + K - 1; i++) {
    const int64_t tau = t0 - (K - 1) + i;
    xr[i] = (tau >= 0 && tau < T) ? load_row<E, V>(x + tau * ldx + c0) : zero_row<E, V>();
  }
  int n = find_seq(cu, N, t0);
  int64_t s = cu[n], e = cu[n + 1];

  if (t0 - (K - 1) >= s && t0 + R <= e && t0 + R <= T) {
    // the run and its K-1 predecessors lie inside one sequence: no masking
#pragma unroll
    for (int r = 0; r < R; r++) {
      float out[V];
#pragma unroll
      for (int i = 0; i < V; i++) {
        float z = bv[i];
#pragma unroll
        for (int j = 0; j < K; j++) z += wv[j][i] * xr[r + j].at(i);
        out[i] = z * fast_sigmoid(z);
      }
      store_row<E, V, true>(y + (t0 + r) * C + c0, out);
    }
    return;
  }

  // runs that touch a sequence start or the batch end: every tap is loaded
  // on its own (L1/L2 hits) with the sequence and halo masks
  Row<E, V> hr[K > 1 ? K - 1 : 1];
  const int64_t cu0 = cu[0];
  const bool use_halo = n_halo > 0 && t0 - (K - 1) < cu0;
#pragma unroll
  for (int i = 0; i < K - 1; i++)
    hr[i] = use_halo ? load_row<E, V>(halo + (int64_t)i * C + c0) : zero_row<E, V>();
#pragma unroll
  for (int r = 0; r < R; r++) {
    const int64_t t = t0 + r;
    if (t < T) {
      while (t >= e) {  // next (non-empty) sequence
        n++;
        s = cu[n];
        e = cu[n + 1];
      }
      float z[V];
#pragma unroll
      for (int i = 0; i < V; i++) z[i] = bv[i];
#pragma unroll
      for (int j = 0; j < K; j++) {
        const int64_t tau = t - (K - 1) + j;
        if (tau >= s) {
          const Row<E, V> xv = load_row<E, V>(x + tau * ldx + c0);
#pragma unroll
          for (int i = 0; i < V; i++) z[i] += wv[j][i] * xv.at(i);
        } else if (n == 0 && s - tau <= n_halo) {
          const int hrow = (int)(K - 1 - (s - tau));
#pragma unroll
          for (int hi = 0; hi < K - 1; hi++)
            if (hi == hrow) {
#pragma unroll
              for (int i = 0; i < V; i++) z[i] += wv[j][i] * hr[hi].at(i);
            }
        }
      }
      float out[V];
#pragma unroll
      for (int i = 0; i < V; i++) out[i] = z[i] * fast_sigmoid(z[i]);
      store_row<E, V, true>(y + t * C + c0, out);
    }
  }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// A thread's run covers tokens [t0, t0+R).  It recomputes z and dz for
// [t0, t0+R+K-1) (the K-1 extra rows feed dx of its last tokens), writes dx
// for its own tokens, the halo gradient when the run holds the start of
// sequence 0, and accumulates dw/dbias over its own tokens.  The rows stream
// through windows of the last K x rows, dz rows and sequence ends: dx of
// token t - (K-1) is formed once dz[t] is known, while the x and dy rows of
// the next few tokens (BwdShape::PD) are already being read.  A block loops over
// token tiles with a fixed grid stride (the grid is at most one round of
// blocks); its four runs' sums are added in LDS and written as one partial
// row, and a second kernel adds the partial rows in a fixed order
// (deterministic dw).
template <typename E, int K, int V>
__global__ __launch_bounds__(kLanes* kRunsPerBlock) __attribute__((amdgpu_waves_per_eu(BwdShape<E>::WAVES)))
void conv_bwd_kernel(
    const E* __restrict__ x, const E* __restrict__ w, const E* __restrict__ bias,
    const E* __restrict__ halo, const int32_t* __restrict__ cu, int N, int64_t T, int C,
    const gdn_cp_meta* __restrict__ meta, const E* __restrict__ dy, E* __restrict__ dx,
    E* __restrict__ dhalo, float* __restrict__ part_w, float* __restrict__ part_b) {
  constexpr int R = kBwdRows;
  constexpr int DR = R + K - 1;  // dz rows t0 .. t0+R+K-2
  constexpr int PD = BwdShape<E>::PD < DR ? BwdShape<E>::PD : DR;
  __shared__ float red[kLanes][V * (K + 1)];
  const int c0 = (blockIdx.y * kLanes + threadIdx.x) * V;
  const bool active = c0 < C;
  const int n_halo = (halo && meta) ? meta->n_halo : 0;

  float dwacc[K][V], dbacc[V];
#pragma unroll
  for (int i = 0; i < V; i++) {
    dbacc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < K; j++) dwacc[j][i] = 0.f;
  }
  // taps and bias kept in the activation type (exact: they are read from it),
  // which leaves registers for the rows in flight.  Every lane reads a valid
  // channel group (an inactive one the first, zeroed after: V > 1 only when V
  // divides C), so the loads are not behind per-lane branches and are in
  // flight together.
  Row<E, V> wv[K], bv;
  const int cw = active ? c0 : 0;
#pragma unroll
  for (int i = 0; i < V; i++) {
    bv.v[i] = bias ? bias[cw + i] : from_f<E>(0.f);
#pragma unroll
    for (int j = 0; j < K; j++) wv[j].v[i] = w[(cw + i) * K + j];
  }
  if (!active) {
    bv = zero_row<E, V>();
#pragma unroll
    for (int j = 0; j < K; j++) wv[j] = zero_row<E, V>();
  }
  const int64_t cu0 = cu[0];

  const int64_t tile_tokens = (int64_t)R * kRunsPerBlock;
  // row t of x or dy, zero outside [0, T): the load reads a valid row (row 0
  // outside; T >= 1 here) and the select zeroes it, so no load sits behind a
  // per-lane branch and the waits count the rows in flight exactly
  auto row_at = [&](const E* base, int64_t t) {
    const bool ok = t >= 0 && t < T;
    const Row<E, V> r = load_row<E, V>(base + (ok ? t : 0) * C + c0);
    return ok ? r : zero_row<E, V>();
  };
  for (int64_t tile = blockIdx.x; active && tile * tile_tokens < T; tile += gridDim.x) {
    const int64_t t0 = tile * tile_tokens + (int64_t)threadIdx.y * R;
    if (t0 >= T) continue;
    // windows: xw[j] = x row t-(K-1)+j, dzw[j] = dz row t-(K-1)+j and ew[j]
    // = the end of that row's sequence, at the current step t
    Row<E, V> xw[K];
    float dzw[K][V];
    int64_t ew[K];
#pragma unroll
    for (int j = 0; j < K; j++) {
      ew[j] = 0;
#pragma unroll
      for (int i = 0; i < V; i++) dzw[j][i] = 0.f;
    }
    xw[0] = zero_row<E, V>();
#pragma unroll
    for (int i = 0; i < K - 1; i++) {
      xw[i + 1] = row_at(x, t0 - (K - 1) + i);
    }

    // the x and dy rows of the next PD tokens are in flight while a row is
    // formed (one row at a time leaves too few bytes in flight per CU)
    Row<E, V> px[PD], pg[PD];
#pragma unroll
    for (int d = 0; d < PD; d++) {
      px[d] = row_at(x, t0 + d);
      pg[d] = row_at(dy, t0 + d);
    }

    int n = find_seq(cu, N, t0);
    int64_t s = cu[n], e = cu[n + 1];
    const int n_first = n;
    const int64_t e_first = e, s_first = s;
#pragma unroll
    for (int r = 0; r < DR; r++) {
      const int64_t t = t0 + r;
#pragma unroll
      for (int j = 0; j + 1 < K; j++) {
        xw[j] = xw[j + 1];
        ew[j] = ew[j + 1];
#pragma unroll
        for (int i = 0; i < V; i++) dzw[j][i] = dzw[j + 1][i];
      }
      xw[K - 1] = px[r % PD];
      const Row<E, V> gr = pg[r % PD];
      if (r + PD < DR) {
        px[r % PD] = row_at(x, t + PD);
        pg[r % PD] = row_at(dy, t + PD);
      }
      if (t < T) {
        while (t >= e) {
          n++;
          s = cu[n];
          e = cu[n + 1];
        }
        ew[K - 1] = e;
        float xt[K][V];  // the taps x~[t-(K-1)+j]
#pragma unroll
        for (int j = 0; j < K; j++) {
          const int64_t tau = t - (K - 1) + j;
#pragma unroll
          for (int i = 0; i < V; i++) xt[j][i] = 0.f;
          if (tau >= s) {
#pragma unroll
            for (int i = 0; i < V; i++) xt[j][i] = xw[j].at(i);
          } else if (n == 0 && s - tau <= n_halo) {
            // a valid halo row (only before local sequence 0; n_halo > 0
            // implies a halo)
            const Row<E, V> hv = load_row<E, V>(halo + (int64_t)(K - 1 - (s - tau)) * C + c0);
#pragma unroll
            for (int i = 0; i < V; i++) xt[j][i] = hv.at(i);
          }
        }
#pragma unroll
        for (int i = 0; i < V; i++) {
          float z = bv.at(i);
#pragma unroll
          for (int j = 0; j < K; j++) z += wv[j].at(i) * xt[j][i];
          const float sg = fast_sigmoid(z);
          const float d = gr.at(i) * sg * (1.f + z * (1.f - sg));
          dzw[K - 1][i] = d;
          if (r < R) {
            dbacc[i] += d;
#pragma unroll
            for (int j = 0; j < K; j++) dwacc[j][i] += d * xt[j][i];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; i++) dzw[K - 1][i] = 0.f;
        ew[K - 1] = t;
      }
      // dx[tp] = sum_j w[j] dz[tp+K-1-j] (= dzw[K-1-j]) over taps inside tp's
      // sequence (whose end is ew[0]), tp = t - (K-1)
      const int rp = r - (K - 1);
      if (rp >= 0 && rp < R) {
        const int64_t tp = t0 + rp;
        if (tp < T) {
          float out[V];
#pragma unroll
          for (int i = 0; i < V; i++) out[i] = 0.f;
#pragma unroll
          for (int j = 0; j < K; j++) {
            if (t - j < ew[0]) {
#pragma unroll
              for (int i = 0; i < V; i++) out[i] += wv[j].at(i) * dzw[K - 1 - j][i];
            }
          }
          store_row<E, V, true>(dx + tp * C + c0, out);
        }
      }
      // halo rows (tokens s0 - i, i = 1..K-1, before local sequence 0) once
      // dz of rows 0 .. K-2 is known: the run starting at cu[0] writes all of
      // them; rows beyond n_halo, or all rows when sequence 0 is empty, get 0
      if (K > 1 && r == K - 2 && dhalo && t0 == cu0) {
        const bool seq0 = (n_first == 0) && (s_first == t0);
#pragma unroll
        for (int i = 1; i < K; i++) {
          float out[V];
#pragma unroll
          for (int v = 0; v < V; v++) out[v] = 0.f;
          if (seq0 && i <= n_halo) {
#pragma unroll
            for (int j = 0; j < K; j++) {
              const int rr = K - 1 - i - j;  // dz row of token s0 - i + K-1-j
              if (rr >= 0 && t0 + rr < e_first) {
#pragma unroll
                for (int v = 0; v < V; v++) out[v] += wv[j].at(v) * dzw[rr + 1][v];
              }
            }
          }
          store_row<E, V>(dhalo + (int64_t)(K - 1 - i) * C + c0, out);
        }
      }
    }
  }
  // block reduction of the four runs (in y order), one partial row per block
  for (int y = 1; y < kRunsPerBlock; y++) {
    if (threadIdx.y == y) {
#pragma unroll
      for (int i = 0; i < V; i++) {
#pragma unroll
        for (int j = 0; j < K; j++) red[threadIdx.x][j * V + i] = dwacc[j][i];
        red[threadIdx.x][K * V + i] = dbacc[i];
      }
    }
    __syncthreads();
    if (threadIdx.y == 0) {
#pragma unroll
      for (int i = 0; i < V; i++) {
#pragma unroll
        for (int j = 0; j < K; j++) dwacc[j][i] += red[threadIdx.x][j * V + i];
        dbacc[i] += red[threadIdx.x][K * V + i];
      }
    }
    __syncthreads();
  }
  if (threadIdx.y == 0 && active) {
#pragma unroll
    for (int i = 0; i < V; i++) {
      if (c0 + i < C) {
#pragma unroll
        for (int j = 0; j < K; j++) part_w[((int64_t)blockIdx.x * C + c0 + i) * K + j] = dwacc[j][i];
        part_b[(int64_t)blockIdx.x * C + c0 + i] = dbacc[i];
      }
    }
  }
}

// dw[c,j] = sum_p part_w[p,c,j] in p order; dbias likewise.  With no tokens
// (P = 0) it writes zeros, the halo gradient included.
template <typename E>
__global__ __launch_bounds__(256) void conv_bwd_finalize_kernel(
    const float* __restrict__ part_w, const float* __restrict__ part_b, int P, int C, int K,
    float* __restrict__ dw, float* __restrict__ dbias, E* __restrict__ dhalo) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t CK = (int64_t)C * K;
  if (idx < CK) {
    float a = 0.f;
    for (int p = 0; p < P; p++) a += part_w[p * CK + idx];
    dw[idx] = a;
  }
  if (dbias && idx < C) {
    float b = 0.f;
    for (int p = 0; p < P; p++) b += part_b[(int64_t)p * C + idx];
    dbias[idx] = b;
  }
  if (P == 0 && dhalo && idx < (int64_t)(K - 1) * C) dhalo[idx] = from_f<E>(0.f);
}

struct ConvArgs {
  const void *x, *w, *bias, *halo;
  const int32_t* cu;
  int N;
  int64_t T;
  int C, K;
  const gdn_cp_meta* meta;
  int64_t ldx;  // token stride of x in elements (forward; C for a contiguous x)
};

template <typename E, int K>
int launch_fwd_k(const ConvArgs& a, void* y, hipStream_t stream) {
  constexpr int VE = Vec16<E>::N;
  const bool vec = (a.C % VE == 0) && (a.ldx % VE == 0) && gdn::aligned16(a.x) &&
                   gdn::aligned16(y) && (a.halo == nullptr || gdn::aligned16(a.halo));
  const int V = vec ? VE : 1;
  const int cvec = (a.C + V - 1) / V;
  dim3 block(kLanes, kRunsPerBlock);
  const int64_t runs = (a.T + kFwdRows - 1) / kFwdRows;
  const int64_t tiles = (runs + kRunsPerBlock - 1) / kRunsPerBlock;
  const int cgroups = (cvec + kLanes - 1) / kLanes;
  if (tiles * cgroups > INT32_MAX) return gdn::fail(GDN_EINVAL, "conv: T * C too large");
  dim3 grid((unsigned)(tiles * cgroups));
  if (vec)
    hipLaunchKernelGGL((conv_fwd_kernel<E, K, VE>), grid, block, 0, stream, (const E*)a.x,
                       (const E*)a.w, (const E*)a.bias, (const E*)a.halo, a.cu, a.N, a.T, a.C,
                       a.ldx, cgroups, a.meta, (E*)y);
  else
    hipLaunchKernelGGL((conv_fwd_kernel<E, K, 1>), grid, block, 0, stream, (const E*)a.x,
                       (const E*)a.w, (const E*)a.bias, (const E*)a.halo, a.cu, a.N, a.T, a.C,
                       a.ldx, cgroups, a.meta, (E*)y);
  return gdn::check_launch("gdn_conv1d_silu_halo");
}

template <typename E>
int launch_fwd(const ConvArgs& a, void* y, hipStream_t stream) {
  switch (a.K) {
    case 1: return launch_fwd_k<E, 1>(a, y, stream);
    case 2: return launch_fwd_k<E, 2>(a, y, stream);
    case 3: return launch_fwd_k<E, 3>(a, y, stream);
    case 4: return launch_fwd_k<E, 4>(a, y, stream);
    case 5: return launch_fwd_k<E, 5>(a, y, stream);
    case 6: return launch_fwd_k<E, 6>(a, y, stream);
    case 7: return launch_fwd_k<E, 7>(a, y, stream);
    case 8: return launch_fwd_k<E, 8>(a, y, stream);
  }
  return gdn::fail(GDN_EINVAL, "conv: K must be in [1, 8]");
}

// token splits of the backward grid: an upper bound, which sizes the workspace
int bwd_splits(int64_t T) {
  const int64_t tile = (int64_t)kBwdRows * kRunsPerBlock;
  int64_t tiles = (T + tile - 1) / tile;
  return (int)(tiles < kBwdMaxSplits ? (tiles < 1 ? 1 : tiles) : kBwdMaxSplits);
}

// the splits a launch uses: no more blocks than run at once (as many four-wave
// blocks a CU as waves a SIMD), since a second, partial round of these
// long-running blocks would keep part of the chip idle
int bwd_launch_splits(int64_t T, int cgroups, int blocks_per_cu) {
  const int cap = bwd_splits(T);
  const int64_t fit = blocks_per_cu * (int64_t)gdn::device_cu_count() / (cgroups > 0 ? cgroups : 1);
  return (int)(fit < 1 ? 1 : (fit < cap ? fit : cap));
}

template <typename E, int K>
int launch_bwd_k(const ConvArgs& a, const void* dy, void* dx, float* dw, float* dbias, void* dhalo,
                 void* ws, hipStream_t stream) {
  constexpr int VE = BwdShape<E>::V;
  const bool vec = (a.C % VE == 0) && gdn::aligned16(a.x) && gdn::aligned16(dy) &&
                   gdn::aligned16(dx) && (a.halo == nullptr || gdn::aligned16(a.halo)) &&
                   (dhalo == nullptr || gdn::aligned16(dhalo));
  const int V = vec ? VE : 1;
  const int cvec = (a.C + V - 1) / V;
  const int cgroups = (cvec + kLanes - 1) / kLanes;
  if (cgroups > 65535) return gdn::fail(GDN_EINVAL, "conv: C too large");
  const int P = a.T > 0 ? bwd_launch_splits(a.T, cgroups, BwdShape<E>::WAVES) : 0;
  float* part_w = (float*)ws;
  float* part_b = part_w + (size_t)P * a.C * K;
  dim3 block(kLanes, kRunsPerBlock);
  dim3 grid(P, cgroups);
  if (P > 0) {
  if (vec)
    hipLaunchKernelGGL((conv_bwd_kernel<E, K, VE>), grid, block, 0, stream, (const E*)a.x,
                       (const E*)a.w, (const E*)a.bias, (const E*)a.halo, a.cu, a.N, a.T, a.C,
                       a.meta, (const E*)dy, (E*)dx, (E*)dhalo, part_w, part_b);
  else
    hipLaunchKernelGGL((conv_bwd_kernel<E, K, 1>), grid, block, 0, stream, (const E*)a.x,
                       (const E*)a.w, (const E*)a.bias, (const E*)a.halo, a.cu, a.N, a.T, a.C,
                       a.meta, (const E*)dy, (E*)dx, (E*)dhalo, part_w, part_b);
  int rc = gdn::check_launch("gdn_conv1d_silu_halo_bwd");
  if (rc != GDN_OK) return rc;
  }
  int64_t work = (int64_t)a.C * K;
  if (work < (int64_t)(K - 1) * a.C) work = (int64_t)(K - 1) * a.C;
  hipLaunchKernelGGL(conv_bwd_finalize_kernel<E>, dim3((unsigned)((work + 255) / 256)), dim3(256), 0,
                     stream, part_w, part_b, P, a.C, K, dw, dbias, (E*)dhalo);
  return gdn::check_launch("gdn_conv1d_silu_halo_bwd(finalize)");
}

template <typename E>
int launch_bwd(const ConvArgs& a, const void* dy, void* dx, float* dw, float* dbias, void* dhalo,
               void* ws, hipStream_t stream) {
  switch (a.K) {
    case 1: return launch_bwd_k<E, 1>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 2: return launch_bwd_k<E, 2>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 3: return launch_bwd_k<E, 3>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 4: return launch_bwd_k<E, 4>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 5: return launch_bwd_k<E, 5>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 6: return launch_bwd_k<E, 6>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 7: return launch_bwd_k<E, 7>(a, dy, dx, dw, dbias, dhalo, ws, stream);
    case 8: return launch_bwd_k<E, 8>(a, dy, dx, dw, dbias, dhalo, ws, stream);
  }
  return gdn::fail(GDN_EINVAL, "conv: K must be in [1, 8]");
}

int validate(const char* fn, const void* x, const void* w, const int32_t* cu, int32_t N, int64_t T,
             int32_t C, int32_t K, const void* y, gdn_dtype dt) {
  if (T < 0 || N < 0) return gdn::fail(GDN_EINVAL, "%s: negative T or N", fn);
  if (C < 1) return gdn::fail(GDN_EINVAL, "%s: C must be >= 1", fn);
  if (K < 1 || K > 8) return gdn::fail(GDN_EINVAL, "%s: K=%d outside [1, 8]", fn, K);
  if (dt != GDN_F32 && dt != GDN_BF16) return gdn::fail(GDN_EINVAL, "%s: unknown dtype", fn);
  if (T > 0 && N < 1) return gdn::fail(GDN_EINVAL, "%s: T > 0 needs N >= 1 sequences", fn);
  if (T > 0 && (!x || !w || !cu || !y)) return gdn::fail(GDN_EINVAL, "%s: null pointer", fn);
  if (T * (int64_t)C >= ((int64_t)1 << 46)) return gdn::fail(GDN_EINVAL, "%s: T*C too large", fn);
  return GDN_OK;
}

}  // namespace

extern "C" int gdn_conv1d_silu_halo(const void* x, const void* w, const void* bias,
                                    const void* halo, const int32_t* cu_seqlens, int32_t N,
                                    int64_t T, int32_t C, int32_t K, const gdn_cp_meta* meta,
                                    void* y, gdn_dtype dt, hipStream_t stream) {
  int rc = validate("gdn_conv1d_silu_halo", x, w, cu_seqlens, N, T, C, K, y, dt);
  if (rc != GDN_OK || T == 0) return rc;
  ConvArgs a{x, w, bias, halo, cu_seqlens, N, T, C, K, meta, C};
  return dt == GDN_BF16 ? launch_fwd<bf16>(a, y, stream) : launch_fwd<float>(a, y, stream);
}

namespace gdn {
// The forward conv reading x with token stride ldx (>= C) elements, e.g. the
// leading C columns of packed projection rows.
int conv_fwd_strided(const void* x, int64_t ldx, const void* w, const void* bias,
                     const void* halo, const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t C,
                     int32_t K, const gdn_cp_meta* meta, void* y, gdn_dtype dt,
                     hipStream_t stream) {
  int rc = validate("conv (strided)", x, w, cu_seqlens, N, T, C, K, y, dt);
  if (rc != GDN_OK || T == 0) return rc;
  if (ldx < C) return fail(GDN_EINVAL, "conv: row stride of x smaller than C");
  ConvArgs a{x, w, bias, halo, cu_seqlens, N, T, C, K, meta, ldx};
  return dt == GDN_BF16 ? launch_fwd<bf16>(a, y, stream) : launch_fwd<float>(a, y, stream);
}
}  // namespace gdn

extern "C" size_t gdn_conv_bwd_workspace_size(int64_t T, int32_t C, int32_t K) {
  if (T <= 0 || C <= 0 || K <= 0) return 0;
  return gdn::round_up((size_t)bwd_splits(T) * (size_t)C * (size_t)(K + 1) * sizeof(float), 256);
}

extern "C" int gdn_conv1d_silu_halo_bwd(const void* x, const void* w, const void* bias,
                                        const void* halo, const int32_t* cu_seqlens, int32_t N,
                                        int64_t T, int32_t C, int32_t K, const gdn_cp_meta* meta,
                                        const void* dy, void* dx, float* dw, float* dbias,
                                        void* dhalo, void* ws, size_t ws_bytes, gdn_dtype dt,
                                        hipStream_t stream) {
  int rc = validate("gdn_conv1d_silu_halo_bwd", x, w, cu_seqlens, N, T, C, K, dx, dt);
  if (rc != GDN_OK) return rc;
  if (!dw) return gdn::fail(GDN_EINVAL, "gdn_conv1d_silu_halo_bwd: dw is null");
  if (T > 0 && !dy) return gdn::fail(GDN_EINVAL, "gdn_conv1d_silu_halo_bwd: dy is null");
  const size_t need = gdn_conv_bwd_workspace_size(T, C, K);
  if (need > 0 && (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)))
    return gdn::fail(GDN_EWORKSPACE,
                     "gdn_conv1d_silu_halo_bwd: workspace needs %zu bytes, 256-byte aligned", need);
  ConvArgs a{x, w, bias, halo, cu_seqlens, N, T, C, K, meta, C};
  return dt == GDN_BF16 ? launch_bwd<bf16>(a, dy, dx, dw, dbias, dhalo, ws, stream)
                        : launch_bwd<float>(a, dy, dx, dw, dbias, dhalo, ws, stream);
}

// ---------------------------------------------------------------------------
// The same backward for callers that cannot allocate: the dw / dbias partial
// rows live in a file-scope device array (one copy per GPU, held until the
// process ends) instead of a caller workspace.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = GDN_CONV_BWD_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this GPU's scratch array, looked up once per device
// with that device current.  In host code the array's name is only a
// stand-in for it, never a device address.
int scratch_for_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return gdn::fail(GDN_EHIP, "gdn_conv1d_silu_halo_bwd_noalloc: no current device below %d",
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gdn::fail(GDN_EHIP, "gdn_conv1d_silu_halo_bwd_noalloc: hipGetSymbolAddress: %s",
                       hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" int gdn_conv1d_silu_halo_bwd_noalloc(const void* x, const void* w, const void* bias,
                                                const void* halo, const int32_t* cu_seqlens,
                                                int32_t N, int64_t T, int32_t C, int32_t K,
                                                const gdn_cp_meta* meta, const void* dy, void* dx,
                                                float* dw, float* dbias, void* dhalo, gdn_dtype dt,
                                                hipStream_t stream) {
  int rc = validate("gdn_conv1d_silu_halo_bwd_noalloc", x, w, cu_seqlens, N, T, C, K, dx, dt);
  if (rc != GDN_OK) return rc;
  const size_t need = gdn_conv_bwd_workspace_size(T, C, K);
  if (need > kScratchBytes)
    return gdn::fail(GDN_EWORKSPACE,
                     "gdn_conv1d_silu_halo_bwd_noalloc: T=%lld C=%d K=%d need %zu bytes of scratch, "
                     "above its fixed %zu; call gdn_conv1d_silu_halo_bwd with a workspace",
                     (long long)T, C, K, need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_for_current_device(&ws)) != GDN_OK) return rc;
  return gdn_conv1d_silu_halo_bwd(x, w, bias, halo, cu_seqlens, N, T, C, K, meta, dy, dx, dw, dbias,
                                  dhalo, ws, kScratchBytes, dt, stream);
}
