// gdn_common.h -- device helpers shared by the libgdn HIP sources (gfx950).
//
// MFMA fragment convention used by every contraction in this library
// ---------------------------------------------------------------------
// A 16x16 output tile C lives in one wave as floatx4 per lane: lane l holds
// C[4*(l/16) + j][l%16] for j = 0..3 (the MFMA accumulator layout).
// The contraction dimension is walked in "k-tiles" of 16.  Inside a k-tile,
// lane group g = l/16 supplies the four k indices 4g..4g+3.  This is the
// same order in which a C tile stores its rows, so an accumulator tile can
// be fed back as the B operand of the next product (K = its row index)
// without moving data between lanes -- the running state S [dk, dv] and the
// corrected values v_new stay in registers between the products of a chunk.
//
//  * bf16 (v_mfma_f32_16x16x32_bf16, K = 32 = two k-tiles): a fragment is 8
//    bf16, elements 0..3 from k-tile 2s, 4..7 from k-tile 2s+1.
//  * fp32 (v_mfma_f32_16x16x4_f32, K = 4): a fragment is one k-tile (4
//    floats); the four MFMAs of a k-tile take element j each.
// A and B supply the same k for the same (lane group, element), so the
// products are exact contractions regardless of the hardware's K order.
// Operands read from LDS are stored [row][k] with k contiguous: A as
// [M][K], B as [N][K] (i.e. B transposed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#define GDN_DEV __device__ __forceinline__

GDN_DEV float to_f(float x) { return x; }
GDN_DEV float to_f(bf16 x) { return (float)x; }

template <typename T> GDN_DEV T from_f(float x);
template <> GDN_DEV float from_f<float>(float x) { return x; }
template <> GDN_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// 16-byte vector of activations.
template <typename E> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  typedef floatx4 type;
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};

template <typename E> GDN_DEV typename Vec16<E>::type zero_vec16() {
  typename Vec16<E>::type z;
#pragma unroll
  for (int i = 0; i < Vec16<E>::N; i++) z[i] = from_f<E>(0.f);
  return z;
}

// ---------------------------------------------------------------------------
// MFMA policy: operand type O of the contractions.
// ---------------------------------------------------------------------------
// Transposed LDS read (ds_read_b64_tr_b16): from a row-major [rows][ld] bf16
// array, lane l (group g = l/16, index i = l%16) receives the four elements
// of column c0 + i in rows r0 + 4g + j, j = 0..3 -- a C-layout tile, or
// half of an A fragment whose contraction index runs down the rows.  Within
// each 16-lane group the instruction returns to lane i element i%4 of the
// 8-byte vector read by lane 4j + i/4, so lane i points at row r0 + 4g +
// i/4, columns c0 + 4(i%4) .. +3.  Addresses must be 8-byte aligned.
typedef short shortx4 __attribute__((ext_vector_type(4)));
// With cs = 8 the four column blocks are c0, c0 + 8, c0 + 16, c0 + 24, and lane
// i receives column c0 + 8(i/4) + i%4 (the permuted dk order of the state).
GDN_DEV bf16x4 lds_rows4_tr(const bf16* base, int ld, int r0, int c0, int lane, int cs = 4) {
  const int i = lane & 15, g = lane >> 4;
  const bf16* p = base + ((4 * g + (i >> 2)) * ld + cs * (i & 3)) + (r0 * ld + c0);
  typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

template <typename O> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 32;  // k per fragment
  typedef bf16x8 frag;

  // rows row0 + l%16 of a [rows][ld] array, k indices k0 + (conv. order)
  GDN_DEV static frag load(const bf16* base, int ld, int row0, int k0, int lane) {
    const bf16* p = base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0);
    bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
    frag f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  }
  // rows row0 + l%16, k indices k0 + 8g .. k0 + 8g + 7 (one 16-byte read): the
  // contraction order of a state whose dk rows are permuted (see dk_of_row)
  GDN_DEV static frag load_k8(const bf16* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + ((lane & 15) * ld + 8 * (lane >> 4)) + (row0 * ld + k0));
  }
  // same from an fp32 [rows][ld] array, element k scaled by sc[k]
  GDN_DEV static frag load_scaled(const float* base, int ld, int row0, int k0, const float* sc,
                                  int lane) {
    const int kl = 4 * (lane >> 4);
    const float* p = base + ((lane & 15) * ld + kl) + (row0 * ld + k0);
    floatx4 lo = *reinterpret_cast<const floatx4*>(p);
    floatx4 hi = *reinterpret_cast<const floatx4*>(p + 16);
    floatx4 slo = *reinterpret_cast<const floatx4*>(sc + kl + k0);
    floatx4 shi = *reinterpret_cast<const floatx4*>(sc + kl + k0 + 16);
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f[j] = (bf16)(lo[j] * slo[j]);
      f[4 + j] = (bf16)(hi[j] * shi[j]);
    }
    return f;
  }
  // same from an fp32 [rows][ld] array (e.g. a state in global memory)
  GDN_DEV static frag load_f32(const float* base, int ld, int row0, int k0, int lane) {
    const float* p = base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0);
    floatx4 lo = *reinterpret_cast<const floatx4*>(p);
    floatx4 hi = *reinterpret_cast<const floatx4*>(p + 16);
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f[j] = (bf16)lo[j];
      f[4 + j] = (bf16)hi[j];
    }
    return f;
  }
  // column access: element (k, c0 + l%16) of a [K][ld] array in LDS, k in
  // the convention's order -- an operand whose contraction index runs down
  // rows; two transposing reads (ld and c0 multiples of 4 elements)
  GDN_DEV static frag load_col(const bf16* base, int ld, int c0, int k0, int lane) {
    const bf16x4 lo = lds_rows4_tr(base, ld, k0, c0, lane);
    const bf16x4 hi = lds_rows4_tr(base, ld, k0 + 16, c0, lane);
    return frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  GDN_DEV static frag load_col_f32(const float* base, int ld, int c0, int k0, const float* sc,
                                   int lane) {
    const int kk = k0 + 4 * (lane >> 4);
    const float* p = base + (4 * (lane >> 4) * ld + (lane & 15)) + (k0 * ld + c0);
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f[j] = (bf16)(sc ? p[j * ld] * sc[kk + j] : p[j * ld]);
      f[4 + j] = (bf16)(sc ? p[(16 + j) * ld] * sc[kk + 16 + j] : p[(16 + j) * ld]);
    }
    return f;
  }
  // column access (LDS, as load_col) with element k scaled by sc[k]
  GDN_DEV static frag load_col_scaled(const bf16* base, int ld, int c0, int k0, const float* sc,
                                      int lane) {
    const int kk = k0 + 4 * (lane >> 4);
    const bf16x4 lo = lds_rows4_tr(base, ld, k0, c0, lane);
    const bf16x4 hi = lds_rows4_tr(base, ld, k0 + 16, c0, lane);
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f[j] = (bf16)((float)lo[j] * sc[kk + j]);
      f[4 + j] = (bf16)((float)hi[j] * sc[kk + 16 + j]);
    }
    return f;
  }
  // B fragment from accumulator tiles of k-tiles 2s and 2s+1
  GDN_DEV static frag from_acc(const floatx4& c0, const floatx4& c1) {
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f[j] = (bf16)c0[j];
      f[4 + j] = (bf16)c1[j];
    }
    return f;
  }
  GDN_DEV static void mma(floatx4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 16;
  typedef floatx4 frag;

  GDN_DEV static frag load(const float* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const floatx4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0));
  }
  GDN_DEV static frag load_scaled(const float* base, int ld, int row0, int k0, const float* sc,
                                  int lane) {
    const int kk = k0 + 4 * (lane >> 4);
    floatx4 a = *reinterpret_cast<const floatx4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0));
    floatx4 s = *reinterpret_cast<const floatx4*>(sc + kk);
    return a * s;
  }
  GDN_DEV static frag load_f32(const float* base, int ld, int row0, int k0, int lane) {
    return load(base, ld, row0, k0, lane);
  }
  GDN_DEV static frag load_col(const float* base, int ld, int c0, int k0, int lane) {
    const float* p = base + (4 * (lane >> 4) * ld + (lane & 15)) + (k0 * ld + c0);
    return frag{p[0], p[ld], p[2 * ld], p[3 * ld]};
  }
  GDN_DEV static frag load_col_scaled(const float* base, int ld, int c0, int k0, const float* sc,
                                      int lane) {
    return load_col_f32(base, ld, c0, k0, sc, lane);
  }
  GDN_DEV static frag load_col_f32(const float* base, int ld, int c0, int k0, const float* sc,
                                   int lane) {
    const int kk = k0 + 4 * (lane >> 4);
    const float* p = base + (4 * (lane >> 4) * ld + (lane & 15)) + (k0 * ld + c0);
    frag f{p[0], p[ld], p[2 * ld], p[3 * ld]};
    if (sc) f *= *reinterpret_cast<const floatx4*>(sc + kk);
    return f;
  }
  GDN_DEV static frag from_acc(const floatx4& c0) { return c0; }
  GDN_DEV static void mma(floatx4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  }
};

// Products over one k-tile (K = 16): bf16 via v_mfma_f32_16x16x16_bf16,
// fp32 via four v_mfma_f32_16x16x4_f32.  Same fragment convention.
template <typename O> struct Tile16;
template <> struct Tile16<bf16> {
  typedef bf16x4 frag;
  // A[row0 + l%16][k0 + 4g .. +3] of a bf16 array
  GDN_DEV static frag load(const bf16* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const bf16x4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0));
  }
  // A[row0 + l%16][k0 + 4g .. +3] of an fp32 array, times s
  GDN_DEV static frag load_f32(const float* base, int ld, int row0, int k0, float s, int lane) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0));
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) f[j] = (bf16)(a[j] * s);
    return f;
  }
  GDN_DEV static frag from_acc(const floatx4& c) {
    frag f;
#pragma unroll
    for (int j = 0; j < 4; j++) f[j] = (bf16)c[j];
    return f;
  }
  GDN_DEV static void mma(floatx4& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
  }
};
template <> struct Tile16<float> {
  typedef floatx4 frag;
  GDN_DEV static frag load(const float* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const floatx4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0));
  }
  GDN_DEV static frag load_f32(const float* base, int ld, int row0, int k0, float s, int lane) {
    return *reinterpret_cast<const floatx4*>(base + ((lane & 15) * ld + 4 * (lane >> 4)) + (row0 * ld + k0)) * s;
  }
  GDN_DEV static frag from_acc(const floatx4& c) { return c; }
  GDN_DEV static void mma(floatx4& acc, const frag& a, const frag& b) { Mfma<float>::mma(acc, a, b); }
};

// The C-layout 16x16 tile at (r0, c0) of a row-major [rows][ld] LDS array,
// as fp32: lane l receives rows r0 + 4(l/16) + j (j = 0..3) of column
// c0 + l%16 (bf16: one transposing read, ld and c0 multiples of 4).
GDN_DEV floatx4 lds_tile_c(const bf16* base, int ld, int r0, int c0, int lane) {
  const bf16x4 v = lds_rows4_tr(base, ld, r0, c0, lane);
  return floatx4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
GDN_DEV floatx4 lds_tile_c(const float* base, int ld, int r0, int c0, int lane) {
  const float* p = base + (r0 + 4 * (lane >> 4)) * ld + c0 + (lane & 15);
  return floatx4{p[0], p[ld], p[2 * ld], p[3 * ld]};
}

GDN_DEV floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

// Make this wave's LDS writes visible to its own later reads from other lanes.
GDN_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for hand-offs through LDS only: waits for this wave's LDS
// operations, not for its global loads and stores in flight (the release
// fence of __syncthreads() would drain those too).  The memory clobber keeps
// the compiler from moving memory operations across it.
GDN_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wave-level butterfly sum over groups of `width` consecutive lanes.
template <int WIDTH> GDN_DEV float group_sum(float v) {
#pragma unroll
  for (int m = WIDTH / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Sum over aligned groups of W <= 16 consecutive lanes with DPP lane moves
// (quad swaps, then the half-row and row mirrors), no LDS round trip.  Every
// lane has a source under these patterns, so bound_ctrl and the zero "old"
// value never take effect; with them the compiler folds each move into its
// add (one v_add_f32_dpp a step instead of a move and an add).
template <int CTRL> GDN_DEV float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int W> GDN_DEV float row_group_sum(float v) {
  static_assert(W == 1 || W == 2 || W == 4 || W == 8 || W == 16, "group of 1..16 lanes");
  if constexpr (W >= 2) v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (W >= 4) v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (W >= 8) v += dpp_mov<0x141>(v);  // row_half_mirror
  if constexpr (W >= 16) v += dpp_mov<0x140>(v); // row_mirror
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves: shifts
// by 1, 2, 4, 8 within each row of 16 lanes (lanes without a source add 0),
// then lane 15 of each row added to the next row and lane 31 to rows 2 and 3.
template <int CTRL, int ROWS, bool BOUND>
GDN_DEV float dpp_upd(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, BOUND));
}
GDN_DEV float wave_incl_scan(float v) {
  v += dpp_upd<0x111, 0xF, true>(v);  // row_shr:1
  v += dpp_upd<0x112, 0xF, true>(v);  // row_shr:2
  v += dpp_upd<0x114, 0xF, true>(v);  // row_shr:4
  v += dpp_upd<0x118, 0xF, true>(v);  // row_shr:8
  v += dpp_upd<0x142, 0xA, false>(v); // row_bcast:15 into rows 1, 3
  v += dpp_upd<0x143, 0xC, false>(v); // row_bcast:31 into rows 2, 3
  return v;
}

// Sum over the whole wave (the inclusive scan's last lane), in every lane.
GDN_DEV float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_scan(v)), 63));
}

// Sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows at one
// position) with the gfx950 row swaps: v_permlane16_swap of a register with
// itself leaves rows (0, 0, 2, 2) and (1, 1, 3, 3), v_permlane32_swap halves
// (lo, lo) and (hi, hi), so each sum of the pair is a sum over the partners.
GDN_DEV float rows4_sum(float v) {
  const unsigned u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float s16 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned w = __float_as_uint(s16);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum of squares of a 16-byte activation vector (bf16: pairwise dot
// products accumulated in fp32).
GDN_DEV float sum_sq(const floatx4& v) { return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]; }
GDN_DEV float sum_sq(const bf16x8& v) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 pr{v[e], v[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, acc, false);
  }
  return acc;
}

// sigmoid with the hardware exp2 and reciprocal (about 1 ulp each)
GDN_DEV float fast_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
