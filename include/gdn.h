/*
 * gdn.h -- C ABI of libgdn, one rank's hot path of a context-parallel Gated
 * DeltaNet token mixer on MI355X (gfx950).
 *
 * Pages cited:
 *   [FLA-CP]  flash-linear-attention "fla/ops/cp/context.py":
 *             get_cp_cu_seqlens, FLACPContext.
 *   [HP-CP]   hyper-parallel "linear_attention_context_parallel.py":
 *             _causal_conv1d_with_cp_halo, _l2norm_torch,
 *             _prepare_gdn_chunks_for_summary, _run_prepared_gdn_chunks,
 *             _RecvInitialStateP2PFunction, _SendFinalStateP2PFunction,
 *             _compute_gdn_state_summary_from_prepared,
 *             the gating lines (beta = sigmoid(b), g = -exp(A_log) softplus(a +
 *             dt_bias)) of the wrappers' forward,
 *             LinearAttentionUlyssesCPWrapper (_seq_to_head_qkvba, its forward),
 *             _merge_gdn_prefix_state_summaries_torch, _apply_gdn_state_summary,
 *             LinearAttentionP2PCPWrapper.forward (the data flow conv ->
 *             split -> GQA expansion -> gated delta rule).
 *
 * General rules for every entry point
 *   - Pointers are device pointers unless stated otherwise.  The caller owns
 *     every buffer, workspaces included; the library allocates no device or
 *     host memory and keeps no state apart from a thread-local error string.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     legacy default stream) and never synchronises the host.  Outputs are
 *     valid once the stream reaches them.
 *   - A call returns GDN_OK or a negative gdn_status without launching
 *     anything when a host-visible argument is invalid; gdn_last_error()
 *     then describes the problem.  Conditions only the device can see (the
 *     contents of cu_seqlens) are reported through gdn_cp_meta.status.
 *   - Activations are `gdn_dtype` (float32 or bfloat16); g, beta, states and
 *     parameter gradients are float32.  Accumulation is float32.
 *   - Concurrent calls on different streams are safe when their buffers
 *     (workspaces included) do not overlap.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_EINVAL = -1,        /* an argument is out of its documented range */
  GDN_EUNSUPPORTED = -2,  /* a valid shape this build has no kernel for */
  GDN_EHIP = -3,          /* a HIP launch or runtime call failed */
  GDN_EWORKSPACE = -4     /* workspace missing or smaller than required */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Device-side status codes written to gdn_cp_meta.status. */
#define GDN_META_OK 0
#define GDN_META_NOT_MONOTONE 1     /* cu_seqlens decreases somewhere */
#define GDN_META_BAD_TOTAL 2        /* cu_seqlens[0] != 0 or cu_seqlens[num_seqs] != total */

/*
 * Per-rank context-parallel record, [FLA-CP] FLACPContext minus the process
 * group.  Lives in device memory; written by gdn_localize_cu_seqlens and read
 * by the conv kernels (n_halo).  Callers that build one by hand (a halo
 * without a shard split) fill it on the host and copy it over.
 */
typedef struct {
  int64_t rank_start;           /* part_len * rank                                  */
  int64_t rank_end;             /* rank_start + part_len                            */
  int64_t pre_num_conv_tokens;  /* max(0, rank_start - start of first local seq)    */
  int32_t num_local_seqs;       /* local sequences (empty pieces dropped)           */
  int32_t first_seq_global_idx; /* global index of local sequence 0                 */
  int32_t is_first_rank;        /* rank owns the first token of local sequence 0    */
  int32_t is_last_rank;         /* rank owns the last token of the last local seq   */
  int32_t pre_num_ranks;        /* ranks before this one holding local sequence 0   */
  int32_t post_num_ranks;       /* ranks after this one holding the last local seq  */
  int32_t n_halo;               /* min(K-1, pre_num_conv_tokens): usable halo rows  */
  int32_t status;               /* GDN_META_* (device-side validation)              */
} gdn_cp_meta;

/*
 * Localise a packed batch to one token shard.  [FLA-CP] get_cp_cu_seqlens,
 * steps 2-5: part_len = total_tokens / world_size, shard
 * [part_len*rank, part_len*(rank+1)); the sequences overlapping it are found
 * by two sorted searches (ends vs rank_start, side right; starts vs rank_end,
 * side left), their boundaries clamped to the shard, rebased and de-duplicated
 * (so empty pieces vanish and local index != global index), then the
 * first/last-owner metadata are derived.  Integer work in int64, bit-exact.
 *
 *   cu_seqlens        int32 [num_seqs+1], non-decreasing, cu[0] = 0,
 *                     cu[num_seqs] = total_tokens.
 *   total_tokens      host copy of cu_seqlens[num_seqs] (as the page reads
 *                     the CPU copy); must be > 0 and divisible by world_size.
 *   conv_kernel_size  K >= 1 of the conv that follows (for n_halo).
 *   local_cu_seqlens  out, int32 [num_seqs+1]: entries 0..num_local_seqs hold
 *                     the local boundaries (0 .. part_len); the remaining
 *                     entries are filled with part_len, so any consumer may
 *                     treat the array as num_seqs sequences, the trailing
 *                     ones empty.
 *   meta              out, one gdn_cp_meta.
 * Errors: GDN_EINVAL for num_seqs < 1, world_size < 1, rank outside
 * [0, world_size), conv_kernel_size < 1, total_tokens <= 0, a remainder
 * (total % world_size != 0, where the page would leave tokens unowned) or
 * null pointers.  A cu_seqlens that is not monotone or does not end at
 * total_tokens sets meta->status (then the other outputs are undefined).
 */
int gdn_localize_cu_seqlens(const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                            int32_t world_size, int32_t rank, int32_t conv_kernel_size,
                            int32_t* local_cu_seqlens, gdn_cp_meta* meta, hipStream_t stream);

/*
 * Causal depthwise conv1d + SiLU with a carried-in halo.  [HP-CP]
 * _causal_conv1d_with_cp_halo: per channel c and token t of sequence n
 * (tokens [cu[n], cu[n+1])):
 *   z[t,c] = bias[c] + sum_{j<K} w[c,j] * xh[t-(K-1)+j, c],   y = z*sigmoid(z)
 * (cross-correlation: w[c,K-1] multiplies the current token).  xh is x inside
 * the token's own sequence; for local sequence 0 the last meta->n_halo rows of
 * `halo` stand for the tokens just before it (halo row K-2 = the token right
 * before); every other position is zero.
 *
 *   x     [T, C] activations, row-major (channels [Q heads|K heads|V heads]).
 *   w     [C, K] activations.          bias [C] activations or NULL.
 *   halo  [K-1, C] activations or NULL (then n_halo is taken as 0).
 *   cu_seqlens int32 [N+1], cu[0] = 0, cu[N] = T (device).
 *   meta  device gdn_cp_meta or NULL (n_halo = 0).
 *   y     [T, C] output; must not overlap x.
 * Errors: GDN_EINVAL for T < 0, N < 0, C < 1, K outside [1, 8], null
 * required pointers or an unknown dtype.  T = 0 launches nothing.
 */
int gdn_conv1d_silu_halo(const void* x, const void* w, const void* bias, const void* halo,
                         const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t C, int32_t K,
                         const gdn_cp_meta* meta, void* y, gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_conv1d_silu_halo_bwd needs for (T, C, K). */
size_t gdn_conv_bwd_workspace_size(int64_t T, int32_t C, int32_t K);

/*
 * Reverse mode of gdn_conv1d_silu_halo.  Given dy = dL/dy [T, C]:
 *   dx    [T, C] activations (overwritten): dL/dx;
 *   dw    [C, K] float32 (overwritten): sum over tokens of dz * xh, reduced
 *         in a fixed order (run-to-run deterministic);
 *   dbias [C] float32 or NULL;
 *   dhalo [K-1, C] activations or NULL: gradient of the halo rows, zero for
 *         the rows beyond n_halo (what the page's differentiable halo
 *         all-to-all hands back to the previous shard).
 * Other arguments as in the forward.  ws/ws_bytes: workspace of at least
 * gdn_conv_bwd_workspace_size(T, C, K) bytes, 256-byte aligned.
 * Errors: as the forward, plus GDN_EWORKSPACE.
 */
int gdn_conv1d_silu_halo_bwd(const void* x, const void* w, const void* bias, const void* halo,
                             const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t C, int32_t K,
                             const gdn_cp_meta* meta, const void* dy, void* dx, float* dw,
                             float* dbias, void* dhalo, void* ws, size_t ws_bytes, gdn_dtype dt,
                             hipStream_t stream);

/* Size of the library's own scratch array used by
 * gdn_conv1d_silu_halo_bwd_noalloc (one per GPU). */
#define GDN_CONV_BWD_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * gdn_conv1d_silu_halo_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the dw / dbias partial rows
 * in a static device array of GDN_CONV_BWD_SCRATCH_BYTES owned by the
 * library (each GPU the library runs on holds its own copy until the process
 * ends) instead of a caller workspace.  The call allocates nothing; the
 * caller still passes every input and output.  The array's device address is
 * looked up once per device, on the first call with that device current.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on different streams, or from several threads without ordering) race and
 * must not be issued; calls ordered on a stream are safe.  Nothing in the
 * array needs to start at zero (each call overwrites the partial rows it
 * reads).
 * Errors: as gdn_conv1d_silu_halo_bwd; GDN_EWORKSPACE when
 * gdn_conv_bwd_workspace_size(T, C, K) exceeds GDN_CONV_BWD_SCRATCH_BYTES
 * (e.g. C above about 13000 channels at K = 4 for long inputs); GDN_EHIP if
 * the array's address cannot be obtained.
 */
int gdn_conv1d_silu_halo_bwd_noalloc(const void* x, const void* w, const void* bias,
                                     const void* halo, const int32_t* cu_seqlens, int32_t N,
                                     int64_t T, int32_t C, int32_t K, const gdn_cp_meta* meta,
                                     const void* dy, void* dx, float* dw, float* dbias,
                                     void* dhalo, gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_chunk_fwd (bwd = 0) or gdn_chunk_bwd (bwd = 1)
 * needs for these sizes; 0 means none. */
size_t gdn_chunk_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                                int32_t dv, gdn_dtype dt, int bwd);

/*
 * Chunked gated delta rule, forward.  [HP-CP] _l2norm_torch,
 * _prepare_gdn_chunks_for_summary, _run_prepared_gdn_chunks, evaluated per
 * sequence of cu_seqlens (sequences never mix; each is chunked in 64-token
 * chunks from its own start).  Per value head h, with q/k head
 * a = h / (Hv/Hk) (the page's repeat_interleave GQA expansion):
 *   qh = scale * q / sqrt(|q|^2 + 1e-6), kh = k / sqrt(|k|^2 + 1e-6)
 *        (plain scale*q, k when use_qk_l2norm = 0);
 *   S <- exp(g_t) S;  S <- S + kh (beta_t (v_t - S^T kh))^T;  o_t = S^T qh
 * with the state S laid out [dk, dv] as the page's recurrent_state, starting
 * from h0[n] (zero if h0 is NULL) and ending as ht[n].
 *
 *   q, k     element (0, head 0, 0) of [T, Hk, dk] views; tokens are ld_qk
 *            elements apart, heads dk apart (e.g. the Q and K channel blocks
 *            of the conv output, ld_qk = C).
 *   v        [T, Hv, dv] view with token stride ld_v.
 *   g, beta  float32 [T, Hv] (g is the per-token log decay, before cumsum).
 *   h0, ht   float32 [N, Hv, dk, dv] or NULL.
 *   cu_seqlens int32 [N+1] (device), cu[0] = 0, cu[N] = T.
 *   scale    multiplier of q (the page uses dk^-1/2).
 *   o        [T, Hv, dv] activations, contiguous.
 *   ws       workspace of gdn_chunk_workspace_size(..., 0) bytes (256-byte
 *            aligned) or NULL when that size is 0.
 * Errors: GDN_EINVAL for negative sizes, Hk < 1, Hv % Hk != 0, ld_qk smaller
 * than Hk*dk, ld_v smaller than Hv*dv, row strides that are not multiples of
 * 16 bytes or whose 64 rows (of q/k, v or o) span 4 GiB or more, null or
 * misaligned required pointers;
 * GDN_EUNSUPPORTED unless dk, dv in {32, 64, 128} (bfloat16) or in {32, 64}
 * (float32, whose chunk tiles would not fit in LDS at 128); GDN_EWORKSPACE.
 */
int gdn_chunk_fwd(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                  const float* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                  int32_t N, int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                  int use_qk_l2norm, void* o, float* ht, void* ws, size_t ws_bytes, gdn_dtype dt,
                  hipStream_t stream);

/*
 * Chunked gated delta rule, backward: reverse mode of gdn_chunk_fwd.  The
 * gradient contract is the page's P2P autograd pair: dht (the final-state
 * gradient coming back from the next shard) in, dh0 (sent to the previous
 * shard) out.  Given d_o [T, Hv, dv] activations and dht [N, Hv, dk, dv]
 * float32 (NULL = zero):
 *   dq, dk_  gradients w.r.t. the raw q, k (before l2norm and scale), summed
 *            over the value heads sharing a q/k head; written through views
 *            with token stride ld_dqk (they may be the Q and K channel blocks
 *            of one [T, C] conv-output gradient).
 *   dv_      [T, Hv, dv] view with token stride ld_dv.
 *   dg, dbeta float32 [T, Hv];  dh0 float32 [N, Hv, dk, dv] or NULL.
 * Forward arguments as in gdn_chunk_fwd.  ws: gdn_chunk_workspace_size(...,1).
 * Errors: the argument checks of gdn_chunk_fwd (GDN_EINVAL, GDN_EWORKSPACE);
 * GDN_EINVAL also for null gradient pointers (d_o, dq, dk_, dv_, dg, dbeta
 * when T > 0), for ld_dqk < Hk*dk or ld_dv < Hv*dv, and when 64 rows of dq,
 * dk or dv (or of the float32 [token, Hv, 2, dk] partial rows kept in the
 * workspace) span 4 GiB or more (a chunk's rows are addressed with 32-bit
 * byte offsets).  The backward has
 * kernels for fewer shapes than the forward: GDN_EUNSUPPORTED unless
 * dk == dv and d is 64 or 128 (bfloat16) or 32 or 64 (float32).
 */
int gdn_chunk_bwd(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                  const float* g, const float* beta, const float* h0, const int32_t* cu_seqlens,
                  int32_t N, int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                  int use_qk_l2norm, const void* d_o, const float* dht, void* dq, void* dk_,
                  int64_t ld_dqk, void* dv_, int64_t ld_dv, float* dg, float* dbeta, float* dh0,
                  void* ws, size_t ws_bytes, gdn_dtype dt, hipStream_t stream);

/* Bytes of the buffer gdn_chunk_fwd_save fills for gdn_chunk_bwd_saved. */
size_t gdn_chunk_saved_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv,
                            gdn_dtype dt);

/*
 * gdn_chunk_fwd that also keeps what gdn_chunk_bwd would otherwise compute
 * again: the state entering every chunk (activations, [chunks][Hv][dk][dv])
 * and, for bfloat16, the prepared per-(chunk, value head) records (T =
 * (I + diag(beta) L)^-1 diag(beta) and the decay factors of the chunk
 * algorithm of [HP-CP] _prepare_gdn_chunks_for_summary).  The training
 * pattern of the page's autograd functions: the forward saves, the backward
 * reads.  o and ht are bit-identical to gdn_chunk_fwd's.
 *
 *   saved   device buffer of gdn_chunk_saved_size(...) bytes, 256-byte
 *           aligned, owned by the caller; its contents are only meaningful
 *           to gdn_chunk_bwd_saved on the same inputs.
 *   other arguments as gdn_chunk_fwd (ws: gdn_chunk_workspace_size(..., 0)).
 * Errors: as gdn_chunk_fwd; GDN_EWORKSPACE also for a null, short or
 * misaligned saved buffer.
 */
int gdn_chunk_fwd_save(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                       const float* g, const float* beta, const float* h0,
                       const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk, int32_t Hv,
                       int32_t dk, int32_t dv, float scale, int use_qk_l2norm, void* o, float* ht,
                       void* saved, size_t saved_bytes, void* ws, size_t ws_bytes, gdn_dtype dt,
                       hipStream_t stream);

/*
 * gdn_chunk_bwd reading the buffer of a gdn_chunk_fwd_save call made with the
 * same q, k, v, g, beta, h0, cu_seqlens, sizes, scale and l2norm flag: the
 * forward pipeline (prep, summaries, per-chunk states) is not run again.
 * Results agree with gdn_chunk_bwd up to rounding (the saved states come
 * from the forward's own segment plan).  Arguments and results as
 * gdn_chunk_bwd (ws: gdn_chunk_workspace_size(..., 1)); saved as above.
 * Errors: as gdn_chunk_bwd; GDN_EINVAL also for a null, short or misaligned
 * saved buffer.  Nothing checks that the buffer belongs to these inputs.
 */
int gdn_chunk_bwd_saved(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                        const float* g, const float* beta, const float* h0,
                        const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk, int32_t Hv,
                        int32_t dk, int32_t dv, float scale, int use_qk_l2norm, const void* d_o,
                        const float* dht, void* dq, void* dk_, int64_t ld_dqk, void* dv_,
                        int64_t ld_dv, float* dg, float* dbeta, float* dh0, const void* saved,
                        size_t saved_bytes, void* ws, size_t ws_bytes, gdn_dtype dt,
                        hipStream_t stream);

/*
 * Gating step.  [HP-CP] LinearAttentionP2PCPWrapper.forward (and the
 * all-gather and Ulysses wrappers), the lines that form the decay and the
 * write strength from the projections: per token t and value head h,
 *     beta[t,h] = sigmoid(b[t,h])
 *     g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 * in float32 (softplus as max(x,0) + log1p(exp(-|x|)), which overflows
 * nowhere; the page's beta is rounded to the activation dtype, here it is
 * kept in float32).
 *
 *   a, b       [T, Hv] activations (dt), token stride ld_ab >= Hv elements
 *              (e.g. two column blocks of packed projection rows).
 *   A_log, dt_bias  float32 [Hv].
 *   g, beta    float32 [T, Hv], contiguous (the gdn_chunk_fwd inputs).
 * Errors: GDN_EINVAL for T < 0, Hv < 1, ld_ab < Hv, an unknown dtype or null
 * pointers when T > 0.
 */
int gdn_gating_fwd(const void* a, const void* b, int64_t ld_ab, const float* A_log,
                   const float* dt_bias, int64_t T, int32_t Hv, float* g, float* beta,
                   gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_gating_bwd needs (per-block partial sums). */
size_t gdn_gating_bwd_workspace_size(int64_t T, int32_t Hv);

/*
 * Reverse mode of gdn_gating_fwd.  Given dg, dbeta float32 [T, Hv]:
 *   db[t,h] = dbeta * beta (1 - beta);
 *   da[t,h] = dg * (-exp(A_log[h])) * sigmoid(a + dt_bias[h]);
 *   ddt_bias[h] = sum_t da[t,h];  dA_log[h] = sum_t dg[t,h] * g[t,h]
 * (sums in a fixed order: run-to-run deterministic).  da, db: activations,
 * token stride ld_dab >= Hv; dA_log, ddt_bias float32 [Hv] or NULL.
 * ws: gdn_gating_bwd_workspace_size(T, Hv) bytes, 256-byte aligned.
 * Errors: as gdn_gating_fwd, plus GDN_EWORKSPACE.
 */
int gdn_gating_bwd(const void* a, const void* b, int64_t ld_ab, const float* A_log,
                   const float* dt_bias, const float* dg, const float* dbeta, int64_t T,
                   int32_t Hv, void* da, void* db, int64_t ld_dab, float* dA_log,
                   float* ddt_bias, void* ws, size_t ws_bytes, gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_chunk_fwd_gated needs for these sizes. */
size_t gdn_chunk_fwd_gated_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                                          int32_t dv, gdn_dtype dt);

/*
 * gdn_chunk_fwd with the gating step fused in: instead of g and beta it
 * takes the projections a, b (activations, [T, Hv] with token stride ld_ab)
 * and A_log, dt_bias (float32 [Hv]), and forms the gates as gdn_gating_fwd
 * does (bit-identical values) where the chunk kernels load them, so g and
 * beta never make a round trip through memory.  g_out / beta_out (float32
 * [T, Hv] or NULL) receive the gates, for a backward.  Other arguments and
 * results as gdn_chunk_fwd; ws: gdn_chunk_fwd_gated_workspace_size(...).
 * Errors: as gdn_chunk_fwd, plus GDN_EINVAL for ld_ab < Hv or null A_log,
 * dt_bias when T > 0.
 */
int gdn_chunk_fwd_gated(const void* q, const void* k, int64_t ld_qk, const void* v, int64_t ld_v,
                        const void* a, const void* b, int64_t ld_ab, const float* A_log,
                        const float* dt_bias, const float* h0, const int32_t* cu_seqlens, int32_t N,
                        int64_t T, int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, float scale,
                        int use_qk_l2norm, void* o, float* ht, float* g_out, float* beta_out,
                        void* ws, size_t ws_bytes, gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_ulysses_fwd needs for these (rank-local) sizes. */
size_t gdn_ulysses_fwd_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                                      int32_t dv, gdn_dtype dt);

/*
 * One rank's forward in the head-sharded (Ulysses) layout.  [HP-CP]
 * LinearAttentionUlyssesCPWrapper: after _seq_to_head_qkvba's all-to-all a
 * rank holds, for the whole (packed) sequence batch, rows
 *     [ q (Hk*dk) | k (Hk*dk) | v (Hv*dv) | b (Hv) | a (Hv) ]
 * of its local heads (Hk, Hv here are the rank's counts: the model's divided
 * by the group size).  It runs the causal conv + SiLU over the local
 * q|k|v channels with the local conv weight slice (the page's
 * _local_conv_weight), forms beta, g from the b, a columns with the local
 * slices of A_log and dt_bias, and the gated delta rule on its heads (GQA
 * v-head h reads q/k head h / (Hv/Hk)).  The q|k|v columns are read in place
 * by the conv and the b|a columns by the chunk kernels' prep; there is no
 * halo (every rank has the whole sequence).
 *
 *   packed     [T, >= 2*Hk*dk + Hv*dv + 2*Hv] activations, token stride
 *              ld_packed elements (16-byte multiples run the vector path).
 *   conv_w     [C, K] activations, C = 2*Hk*dk + Hv*dv (the rank's slice);
 *              conv_bias [C] or NULL.  K in [1, 8].
 *   A_log, dt_bias  float32 [Hv] (the rank's slices).
 *   h0, ht     float32 [N, Hv, dk, dv] or NULL (the page passes none).
 *   y          out, [T, C] activations: the conv output (q, k, v of the
 *              chunk; keep it for a backward).
 *   o          out, [T, Hv, dv] activations.
 *   g_out, beta_out  float32 [T, Hv] or NULL: the gates, for a backward.
 *   ws         gdn_ulysses_fwd_workspace_size(...) bytes, 256-byte aligned.
 * Errors: GDN_EINVAL for ld_packed < C + 2*Hv, null pointers and the checks
 * of gdn_conv1d_silu_halo and gdn_chunk_fwd_gated; GDN_EUNSUPPORTED and
 * GDN_EWORKSPACE as gdn_chunk_fwd_gated.  Nothing is launched when a check
 * fails.
 */
int gdn_ulysses_fwd(const void* packed, int64_t ld_packed, const void* conv_w,
                    const void* conv_bias, int32_t K, const float* A_log, const float* dt_bias,
                    const float* h0, const int32_t* cu_seqlens, int32_t N, int64_t T, int32_t Hk,
                    int32_t Hv, int32_t dk, int32_t dv, float scale, int use_qk_l2norm, void* y,
                    void* o, float* ht, float* g_out, float* beta_out, void* ws, size_t ws_bytes,
                    gdn_dtype dt, hipStream_t stream);

/* Bytes of workspace gdn_chunk_summary needs for these sizes. */
size_t gdn_chunk_summary_workspace_size(int64_t T, int32_t N, int32_t Hk, int32_t Hv, int32_t dk,
                                        int32_t dv, gdn_dtype dt);

/*
 * Affine state summary of every local sequence of a shard.  [HP-CP]
 * _compute_gdn_state_summary_from_prepared: the gated delta rule of
 * gdn_chunk_fwd is affine in its initial state, so for each sequence n and
 * value head h the state leaving it is
 *     S_out = M[n,h] S_in + E[n,h],
 * M [dk, dk] the product of the chunk transitions e^{G_C} I - (kh o
 * e^{G_C - G})^T w and E [dk, dv] the state reached from S_in = 0.  This is
 * what a rank computes before it knows its carried-in state (the page's P2P
 * wavefront and all-gather modes exchange it).  An empty sequence gives
 * M = I, E = 0.  q plays no part; scale is irrelevant.
 *
 *   k, v, g, beta, cu_seqlens, N, T, Hk, Hv, dk, dv, use_qk_l2norm, dt: as
 *            in gdn_chunk_fwd (k with token stride ld_k).
 *   M        float32 [N, Hv, dk, dk] or NULL (not written).
 *   E        float32 [N, Hv, dk, dv] or NULL (not written).
 *   ws       gdn_chunk_summary_workspace_size(...) bytes, 256-byte aligned.
 * Errors: as gdn_chunk_fwd (shapes, strides, dtypes, workspace); GDN_EINVAL
 * also for M or E not 16-byte aligned.
 */
int gdn_chunk_summary(const void* k, int64_t ld_k, const void* v, int64_t ld_v, const float* g,
                      const float* beta, const int32_t* cu_seqlens, int32_t N, int64_t T,
                      int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, int use_qk_l2norm, float* M,
                      float* E, void* ws, size_t ws_bytes, gdn_dtype dt, hipStream_t stream);

/*
 * Prefix merge of affine summaries.  [HP-CP]
 * _merge_gdn_prefix_state_summaries_torch (fold the summaries of the ranks
 * before this one from a zero state) and _apply_gdn_state_summary (one
 * summary applied to a received state): for every state slot s (e.g. a
 * (sequence, value head) pair),
 *     h = h_in[s] (zero if h_in is NULL);  h <- M[r,s] h + E[r,s] for r = 0 .. R-1;
 *     h_out[s] = h.
 *
 *   M      float32 [R, S, dk, dk];  E float32 [R, S, dk, dv]  (R >= 0).
 *   h_in   float32 [S, dk, dv] or NULL;  h_out float32 [S, dk, dv] (may be
 *          h_in: each workgroup reads its columns before it writes them).
 * fp32 arithmetic (MFMA).  Errors: GDN_EINVAL for negative R or S, null or
 * non-16-byte-aligned pointers; GDN_EUNSUPPORTED unless dk, dv in
 * {32, 64, 128}.
 */
int gdn_merge_summaries(const float* M, const float* E, int32_t R, int32_t S, int32_t dk,
                        int32_t dv, const float* h_in, float* h_out, hipStream_t stream);

/* Thread-local description of the last non-OK status ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
