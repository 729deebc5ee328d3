// chunk_plan.h -- device-side work lists of the chunk kernels (no host sync).
//
// From cu_seqlens one workgroup derives, for every sequence n (each chunked
// in 64-token chunks from its own start):
//   * its segments: a first run of `seg_first` tokens, then runs of `seg_len`
//     tokens, each handled by one workgroup
//     (table[s] = {n, token begin, token end, first/last flags}, seg_chunk0[s]
//     = global index of the segment's first chunk);
//   * seq_off[n] / seq_nseg[n]: its first segment and segment count;
//   * seq_chunk_off[n]: the global index of its first chunk;
//   * chunk_tab[c] = {chunk begin token, end token of its sequence, n}.
// Counts go to counts[0] (segments) and counts[1] (chunks).  Capacities are
// host-side upper bounds (T / seg_len + N segments, T / 64 + N chunks); the
// kernels size their grids by them and exit past the counts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "gdn_internal.h"

namespace gdn_chunk {

constexpr int kFirst = 1, kLast = 2;

struct PlanPtrs {
  int32_t* counts;  // [2]
  int4* table;      // [seg_cap]
  int32_t* seg_chunk0;
  int32_t* seq_off;
  int32_t* seq_nseg;
  int32_t* seq_chunk_off;
  int4* chunk_tab;  // [chunk_cap] (may be null)
};

namespace {

__device__ __forceinline__ int block_excl_scan256(int v, int* buf, int* total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  const int incl = buf[t];
  *total = buf[255];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int N, int64_t T,
                                                   int seg_first, int seg_len, int seg_cap,
                                                   int chunk_cap, PlanPtrs pp) {
  __shared__ int buf[256];
  __shared__ int sc_off[257];     // chunk offsets of this block's sequences (block-local)
  __shared__ int sc_beg[256], sc_end[256];
  const int t = threadIdx.x;
  int run_seg = 0, run_chunk = 0;
  for (int base = 0; base < N; base += 256) {
    const int n = base + t;
    int64_t s = 0, e = 0;
    int ns = 0, nc = 0;
    if (n < N) {
      s = cu[n];
      e = cu[n + 1];
      s = s < 0 ? 0 : (s > T ? T : s);
      e = e < s ? s : (e > T ? T : e);
      ns = e - s <= seg_first ? (e > s ? 1 : 0) : 1 + (int)((e - s - seg_first + seg_len - 1) / seg_len);
      nc = (int)((e - s + 63) / 64);
    }
    int tot_s = 0, tot_c = 0;
    const int off_s = run_seg + block_excl_scan256(ns, buf, &tot_s);
    const int off_c = run_chunk + block_excl_scan256(nc, buf, &tot_c);
    if (n < N) {
      pp.seq_off[n] = off_s;
      pp.seq_nseg[n] = ns;
      pp.seq_chunk_off[n] = off_c;
      for (int p = 0; p < ns && off_s + p < seg_cap; p++) {
        const int64_t a = p == 0 ? s : s + seg_first + (int64_t)(p - 1) * seg_len;
        const int64_t len = p == 0 ? seg_first : seg_len;
        const int64_t b = a + len < e ? a + len : e;
        pp.table[off_s + p] =
            make_int4(n, (int)a, (int)b, (p == 0 ? kFirst : 0) | (p == ns - 1 ? kLast : 0));
        pp.seg_chunk0[off_s + p] = off_c + (p == 0 ? 0 : (seg_first + (p - 1) * seg_len) / 64);
      }
    }
    if (pp.chunk_tab) {
      // the chunk table of these (up to) 256 sequences, filled by all threads:
      // entry c of the block belongs to the sequence whose block-local range
      // [sc_off[i], sc_off[i + 1]) holds it (binary search)
      sc_off[t] = off_c - run_chunk;
      sc_beg[t] = (int)s;
      sc_end[t] = (int)e;
      if (t == 0) sc_off[256] = tot_c;
      __syncthreads();
      const int nseq = N - base < 256 ? N - base : 256;
      for (int c = t; c < tot_c; c += 256) {
        int lo = 0, hi = nseq - 1;  // last i with sc_off[i] <= c
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sc_off[mid] <= c) lo = mid;
          else hi = mid - 1;
        }
        const int gc = run_chunk + c;
        if (gc < chunk_cap)
          pp.chunk_tab[gc] = make_int4(sc_beg[lo] + 64 * (c - sc_off[lo]), sc_end[lo], base + lo, 0);
      }
      __syncthreads();
    }
    run_seg += tot_s;
    run_chunk += tot_c;
  }
  if (t == 0) {
    pp.counts[0] = run_seg < seg_cap ? run_seg : seg_cap;
    pp.counts[1] = run_chunk < chunk_cap ? run_chunk : chunk_cap;
  }
}

}  // namespace

// Host-side layout of the plan inside a workspace.
struct Plan {
  int64_t seg_first, seg_len;
  // segment indices a state-pass launch covers (its grid)
  int64_t seg_span;
  int64_t seg_cap, chunk_cap;
  bool split;  // some sequence may have more than one segment
  size_t off_counts, off_table, off_seg_chunk0, off_seq_off, off_seq_nseg, off_seq_chunk_off,
      off_chunk_tab, off_state, off_init, off_rec, off_warm, off_seq_warm, end;

  PlanPtrs ptrs(char* ws, bool with_chunks) const {
    PlanPtrs p;
    p.counts = reinterpret_cast<int32_t*>(ws + off_counts);
    p.table = reinterpret_cast<int4*>(ws + off_table);
    p.seg_chunk0 = reinterpret_cast<int32_t*>(ws + off_seg_chunk0);
    p.seq_off = reinterpret_cast<int32_t*>(ws + off_seq_off);
    p.seq_nseg = reinterpret_cast<int32_t*>(ws + off_seq_nseg);
    p.seq_chunk_off = reinterpret_cast<int32_t*>(ws + off_seq_chunk_off);
    p.chunk_tab = with_chunks ? reinterpret_cast<int4*>(ws + off_chunk_tab) : nullptr;
    return p;
  }
};

// Segment lengths from the device size and the number of (sequence, head)
// chains (a test hook on the calling thread can force them).  rec_bytes: bytes of the
// prepared record per (chunk, value head), 0 when the state pass takes none.
// summaries: the plan of a shard summary, which keeps every segment's [M | E].
//
// A state-pass workgroup takes most of a CU's LDS, so one runs per CU.  Each
// XCD hands its share of a grid (ids x mod 8 go to XCD x) to its CUs in a
// fixed rotation, also the workgroups that exit at once: more than one
// workgroup per CU in a grid can put two long-running ones on one CU.  For a
// single sequence the grids therefore hold exactly CUs / Hv segment indices a
// head, equal segments.
inline Plan make_plan(int64_t T, int32_t N, int32_t Hv, int32_t dk, int32_t dv, size_t rec_bytes,
                      bool summaries = false) {
  Plan p{};
  const int64_t chunks = (T + 63) / 64 + N;  // bound on chunk count over all sequences
  int64_t per = 1, span = 0;
  const int forced = gdn::segment_chunks_override();
  const int64_t C = (T + 63) / 64 + N - 1;
  const int64_t cus = gdn::device_cu_count();
  if (forced > 0) {
    per = forced;
  } else if (N == 1) {
    const int64_t B = cus / Hv > 1 ? cus / Hv : 1;
    per = C > B ? (C + B - 1) / B : 1;
    span = C > 0 ? (C + per - 1) / per : 1;
  } else {
    // several sequences: segments per head at most ceil(C / per) + N - 1
    const int64_t slots = cus * 15 / 16;
    const int64_t budget = slots / Hv > 1 ? slots / Hv : 1;
    per = budget > N ? (C + (budget - N + 1) - 1) / (budget - N + 1) : C + 1;
    if (per < 1) per = 1;
  }
  p.seg_first = per * 64;
  p.seg_len = per * 64;
  p.split = p.seg_first < T;
  if (N == 1 && span > 0) {
    p.seg_cap = span;
  } else {
    p.seg_cap = T / p.seg_len + N + 2;
  }
  p.seg_span = p.seg_cap;
  p.chunk_cap = chunks + 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = gdn::round_up(o + bytes, 256);
    return at;
  };
  p.off_counts = take(8);
  p.off_table = take(sizeof(int4) * (size_t)p.seg_cap);
  p.off_seg_chunk0 = take(4 * (size_t)p.seg_cap);
  p.off_seq_off = take(4 * (size_t)N);
  p.off_seq_nseg = take(4 * (size_t)N);
  p.off_seq_chunk_off = take(4 * (size_t)N);
  p.off_chunk_tab = take(sizeof(int4) * (size_t)p.chunk_cap);
  // summaries: every segment's [M | E] is kept (a shard's summary), split or not
  p.off_state = take(p.split || summaries ? sizeof(float) * (size_t)p.seg_cap * Hv * dk * (dk + dv) : 0);
  p.off_init = take(p.split ? sizeof(float) * (size_t)p.seg_cap * Hv * dk * dv : 0);
  p.off_rec = take(rec_bytes * (size_t)p.chunk_cap * Hv);
  // replay lengths per (segment, head) and the per-(sequence, head) choice
  // of the replay over the summaries (prepared path, split sequences)
  const bool warm = rec_bytes > 0 && p.split;
  p.off_warm = take(warm ? 4 * (size_t)p.seg_cap * Hv : 0);
  p.off_seq_warm = take(warm ? 4 * (size_t)N * Hv : 0);
  p.end = o;
  return p;
}

}  // namespace gdn_chunk
