// localize.hip -- cu_seqlens localisation to one token shard.
//
// flash-linear-attention "fla/ops/cp/context.py", get_cp_cu_seqlens (its
// steps 2-5), on the device so a captured or host-free pipeline needs no D2H
// copy.  One workgroup; all arithmetic in int64.  For a non-decreasing array
// a sorted search is a count: searchsorted(a, v, right) = #{a_i <= v} and
// searchsorted(a, v, left) = #{a_i < v}, so both searches are block-wide
// counts.  The de-duplication (unique_consecutive) is a block-wide stream
// compaction with an exclusive scan.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  int64_t r = red[0];
  __syncthreads();
  return r;
}

// Exclusive scan of one flag per thread; returns the prefix, *total the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* buf, int* total) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  int incl = buf[t];
  *total = buf[kThreads - 1];
  __syncthreads();
  return incl - v;
}

__global__ __launch_bounds__(kThreads) void localize_kernel(const int32_t* __restrict__ cu,
                                                            int32_t num_seqs, int64_t total,
                                                            int32_t world_size, int32_t rank,
                                                            int32_t conv_k, int32_t* __restrict__ local_cu,
                                                            gdn_cp_meta* __restrict__ meta) {
  __shared__ int64_t red[kThreads];
  __shared__ int scan_buf[kThreads];
  const int t = threadIdx.x;
  const int64_t part_len = total / world_size;
  const int64_t rank_start = part_len * rank;
  const int64_t rank_end = rank_start + part_len;

  // validation: cu[0] == 0, cu[num_seqs] == total, non-decreasing
  int64_t bad = 0;
  for (int i = t; i < num_seqs; i += kThreads)
    if (cu[i + 1] < cu[i]) bad = 1;
  const int64_t n_bad = block_sum(bad, red);
  const bool bad_total = (cu[0] != 0) || ((int64_t)cu[num_seqs] != total);

  // start_seq_idx = #{ends cu[1..n] <= rank_start}; end_seq_idx = #{starts cu[0..n-1] < rank_end}
  int64_t c_start = 0, c_end = 0;
  for (int i = t; i < num_seqs; i += kThreads) {
    c_start += ((int64_t)cu[i + 1] <= rank_start);
    c_end += ((int64_t)cu[i] < rank_end);
  }
  const int64_t start_idx = block_sum(c_start, red);
  const int64_t end_idx = block_sum(c_end, red);

  // clamp, rebase and drop consecutive repeats of cu[start_idx..end_idx]
  const int64_t m = end_idx - start_idx + 1;
  int64_t written = 0;
  for (int64_t base = 0; base < m; base += kThreads) {
    const int64_t i = base + t;
    int64_t val = 0;
    int keep = 0;
    if (i < m) {
      int64_t c = cu[start_idx + i];
      c = c < rank_start ? rank_start : (c > rank_end ? rank_end : c);
      val = c - rank_start;
      if (i == 0) {
        keep = 1;
      } else {
        int64_t p = cu[start_idx + i - 1];
        p = p < rank_start ? rank_start : (p > rank_end ? rank_end : p);
        keep = (p - rank_start) != val;
      }
    }
    int tile_total = 0;
    const int pos = block_exclusive_scan(keep, scan_buf, &tile_total);
    if (keep) local_cu[written + pos] = (int32_t)val;
    written += tile_total;
  }
  // pad: the trailing entries describe empty sequences at the shard end
  for (int64_t i = written + t; i <= num_seqs; i += kThreads) local_cu[i] = (int32_t)part_len;

  if (t == 0) {
    const int64_t first_start = cu[start_idx];
    const int64_t last_end = cu[end_idx];
    int64_t pre_conv = rank_start - first_start;
    if (pre_conv < 0) pre_conv = 0;
    const int64_t first_rank = first_start / part_len;
    const int64_t last_rank = (last_end - 1) / part_len;
    const int64_t halo_rows = conv_k > 1 ? conv_k - 1 : 0;
    gdn_cp_meta mt;
    mt.rank_start = rank_start;
    mt.rank_end = rank_end;
    mt.pre_num_conv_tokens = pre_conv;
    mt.num_local_seqs = (int32_t)(written - 1);
    mt.first_seq_global_idx = (int32_t)start_idx;
    mt.is_first_rank = rank == first_rank;
    mt.is_last_rank = rank == last_rank;
    mt.pre_num_ranks = (int32_t)(rank - first_rank);
    mt.post_num_ranks = (int32_t)(last_rank - rank);
    mt.n_halo = (int32_t)(pre_conv < halo_rows ? pre_conv : halo_rows);
    mt.status = n_bad ? GDN_META_NOT_MONOTONE : (bad_total ? GDN_META_BAD_TOTAL : GDN_META_OK);
    *meta = mt;
  }
}

}  // namespace

extern "C" int gdn_localize_cu_seqlens(const int32_t* cu_seqlens, int32_t num_seqs,
                                       int64_t total_tokens, int32_t world_size, int32_t rank,
                                       int32_t conv_kernel_size, int32_t* local_cu_seqlens,
                                       gdn_cp_meta* meta, hipStream_t stream) {
  using gdn::fail;
  if (!cu_seqlens || !local_cu_seqlens || !meta)
    return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: null pointer");
  if (num_seqs < 1) return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: num_seqs must be >= 1");
  if (world_size < 1) return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: world_size must be >= 1");
  if (rank < 0 || rank >= world_size)
    return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: rank %d outside [0, %d)", rank, world_size);
  if (conv_kernel_size < 1)
    return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: conv_kernel_size must be >= 1");
  if (total_tokens <= 0 || total_tokens > INT32_MAX)
    return fail(GDN_EINVAL, "gdn_localize_cu_seqlens: total_tokens %lld outside (0, 2^31)",
                (long long)total_tokens);
  if (total_tokens % world_size != 0)
    return fail(GDN_EINVAL,
                "gdn_localize_cu_seqlens: total_tokens %lld is not divisible by world_size %d",
                (long long)total_tokens, world_size);
  hipLaunchKernelGGL(localize_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, num_seqs,
                     total_tokens, world_size, rank, conv_kernel_size, local_cu_seqlens, meta);
  return gdn::check_launch("gdn_localize_cu_seqlens");
}
