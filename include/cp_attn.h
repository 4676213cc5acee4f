/*
 * cp_attn.h -- C ABI of libcpattn: the per-rank hot path of context-parallel
 * causal attention on AMD Instinct MI355X (gfx950).
 *
 * The operations, and where the pages define them:
 *
 *   cp_shard_plan     which new tokens a CP rank owns, in what local order,
 *                     with what positions and causal KV extents.
 *                     "Prefill Context Parallelism" (SGLang docs), sections
 *                     "Zigzag strategy" and "Interleave strategy".
 *   cp_restore_index  the permutation that puts the rank-major all-gathered
 *                     token order back into causal order.  "What is Context
 *                     Parallelism" (blog), sections 2.1 and 5.1.
 *   cp_restore_apply  that permutation applied on the GPU (a row gather).
 *   cp_choose_pass    pass-KV or pass-Q for a request mix, and
 *   cp_ring_pad_len   the padded ring message length.  Same blog, section 3.5.
 *   cp_attn_fwd       causal attention of one rank's query rows against a KV
 *                     buffer (the gathered KV, one ring round's KV block, or
 *                     one decode shard), giving the normalised output O and
 *                     its log-sum-exp L.  Same blog, sections 2.1, 3.1-3.3;
 *                     GQA head sharing section 4.1, MLA latent section 4.2.
 *   cp_lse_merge      merge of partial (O_j, L_j) into the exact result.
 *                     Same blog, section 3.6.
 *
 * Conventions shared by every call:
 *   - Ownership: the caller owns every buffer (host and device) and the
 *     stream.  The library allocates no device memory; scratch comes from a
 *     caller workspace whose size cp_attn_workspace_size reports, or, for
 *     cp_attn_fwd_noalloc, from a static device array inside the library.
 *     Between calls it keeps only the text of the calling thread's last
 *     error (thread-local, read by cp_last_error) and each GPU's address of
 *     that static array; no result of a call depends on an earlier call.
 *   - Errors: every call returns a cp_status and never throws.  Arguments
 *     are checked on the host before anything is enqueued; on an error
 *     nothing is enqueued.  CP_ERR_SMALL_BUFFER still writes the required
 *     sizes to the size outputs.
 *   - Asynchrony: the GPU calls only enqueue work on `stream` (a hipStream_t
 *     passed as void*; NULL is the null stream).  The caller synchronises.
 *   - Determinism: planner outputs are pure functions of the inputs; a GPU
 *     call with the same inputs is bitwise repeatable.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CP_OK = 0,
  CP_ERR_ARG = 1,          /* an argument is out of range or inconsistent  */
  CP_ERR_UNSUPPORTED = 2,  /* valid, but no kernel for this shape/dtype     */
  CP_ERR_SMALL_BUFFER = 3, /* an output capacity is too small               */
  CP_ERR_DEVICE = 4        /* the HIP runtime reported an error at launch   */
} cp_status;

typedef enum { CP_ZIGZAG = 0, CP_INTERLEAVE = 1 } cp_strategy;

typedef enum { CP_F32 = 0, CP_BF16 = 1 } cp_dtype;

/*
 * One segment: a run of a rank's local query rows that belong to one request
 * and whose positions form an arithmetic sequence.  Zigzag gives one segment
 * per owned non-empty block (early block, then late block, per request);
 * interleave gives one segment per request the rank owns tokens of.
 *
 *   req         request index in the batch
 *   q_begin     first local row; q_end one past the last
 *   pos_begin   absolute position of row q_begin (cached prefix included)
 *   pos_stride  position step between consecutive rows (1 zigzag, C interleave)
 *   kv_begin    first row of the request in the KV buffer
 *   kv_end      one past the last KV row the segment can see: the request's
 *               rows are packed prefix then new tokens, so for the gathered
 *               KV this is kv_begin + (last row's position) + 1.  This is the
 *               block's own "kv length" that the zigzag metadata records.
 */
typedef struct {
  int32_t req, q_begin, q_end, pos_begin, pos_stride, kv_begin, kv_end;
} cp_segment;

/*
 * cp_shard_plan -- host only, integer.
 * "Prefill Context Parallelism", "Zigzag strategy": each request's new
 * tokens are cut into 2C contiguous blocks, the first (T mod 2C) blocks one
 * token longer; rank r owns blocks r and 2C-1-r; the cut restarts per
 * request.  "Interleave strategy": rank r owns flattened new-token indices
 * g = r, r+C, r+2C, ... counted over the whole batch without reset.
 * Positions keep their original values (prefix_b + offset).
 *
 * In:  strategy (cp_strategy), cp_size C >= 1, 0 <= cp_rank < C,
 *      num_reqs >= 0, new_lens[num_reqs] >= 0, prefix_lens[num_reqs] >= 0
 *      (prefix_lens may be NULL: all zero).  All host pointers.
 * Out (each optional, NULL = not wanted):
 *      segs[seg_cap]          the rank's segments, in local row order
 *      *num_segs              number of segments
 *      positions[tok_cap]     absolute position of each local row
 *      global_idx[tok_cap]    flattened new-token index of each local row
 *      *num_local             number of local rows N_r
 *      *padded_local          max over ranks of N_r (the per-rank slice length
 *                             of the padded, all-gathered buffer)
 * Errors: CP_ERR_ARG for a bad strategy, C, rank or negative length, or
 *      int32 overflow of a total; CP_ERR_SMALL_BUFFER when a non-NULL array
 *      is shorter than needed (the size outputs are still written).
 */
cp_status cp_shard_plan(int32_t strategy, int32_t cp_size, int32_t cp_rank,
                        int32_t num_reqs, const int32_t *new_lens,
                        const int32_t *prefix_lens, cp_segment *segs,
                        int32_t seg_cap, int32_t *num_segs, int32_t *positions,
                        int32_t *global_idx, int32_t tok_cap,
                        int32_t *num_local, int32_t *padded_local);

/*
 * cp_restore_index -- host only, integer.
 * The all-gathered buffer holds rank 0's N_0 local rows padded to
 * padded_local slots, then rank 1's, and so on (C * padded_local slots).
 * restore[g] is the slot of flattened new token g, so gathering the buffer
 * by `restore` yields causal (flattened batch) order.  Padding slots are
 * never referenced.
 * In:  strategy, cp_size, num_reqs, new_lens (host).
 * Out: restore[cap] (optional), *padded_local (optional).
 * Errors: as cp_shard_plan; CP_ERR_SMALL_BUFFER if cap < sum(new_lens).
 */
cp_status cp_restore_index(int32_t strategy, int32_t cp_size, int32_t num_reqs,
                           const int32_t *new_lens, int32_t *restore,
                           int32_t cap, int32_t *padded_local);

/*
 * cp_restore_apply -- device gather: dst row i = src row index[i], i < n
 * ("What is Context Parallelism", section 2.1 engineering notes and section
 * 5.1: the rank-major all-gathered buffer, gathered by the restore index,
 * is in causal order).  Enqueued on `stream` (a hipStream_t, NULL = the
 * default stream); the caller owns every buffer.
 * In:  index   DEVICE int32[n]; an entry outside [0, src_rows) zero-fills
 *              its dst row (nothing is read out of bounds);
 *      src     DEVICE, src_rows rows of row_bytes bytes, src_row_stride
 *              bytes apart;
 *      dst     DEVICE, n rows, dst_row_stride bytes apart (must not overlap
 *              src);
 *      row_bytes, both strides and both base pointers: multiples of 16, each
 *      stride >= row_bytes.
 * Errors: CP_ERR_ARG (negative sizes, NULL pointers, alignment or stride),
 * CP_ERR_DEVICE (launch failed).  n = 0 or row_bytes = 0 enqueues nothing.
 */
cp_status cp_restore_apply(const int32_t *index, int64_t n, const void *src, int64_t src_rows,
                           int64_t src_row_stride, void *dst, int64_t dst_row_stride,
                           int64_t row_bytes, void *stream);

/*
 * cp_choose_pass -- host only.  Which ring variant moves less data
 * ("What is Context Parallelism", section 3.5, pass-KV / pass-Q switch):
 * with miss rate T / (T + P), pass-Q when T / (T + P) <= 2 * n_kv_heads /
 * n_heads (compared exactly in integers), else pass-KV.
 * In:  new_tokens T >= 1, cached_tokens P >= 0 (each <= 2^48),
 *      1 <= n_kv_heads <= n_heads.
 * Out (each optional): *pass (cp_pass), *miss_rate, *h_score = the section's
 *      empirical fit -1.059 ln T + 1.145 ln(T/(T+P)) + 12.112 (h > 0
 *      favours pass-KV; informational, it does not decide *pass).
 * Errors: CP_ERR_ARG.
 */
typedef enum { CP_PASS_KV = 0, CP_PASS_Q = 1 } cp_pass;
cp_status cp_choose_pass(int64_t new_tokens, int64_t cached_tokens, int32_t n_heads,
                         int32_t n_kv_heads, int32_t *pass, double *miss_rate, double *h_score);

/*
 * cp_ring_pad_len -- host only.  Length every rank pads its ring message to
 * (same section: max_i P_i + ceil(T / N) with P_i the tokens cached on rank i
 * and T the new tokens over N = cp_size ranks).
 * In:  cp_size >= 1, cached_per_rank (host, cp_size entries >= 0),
 *      new_tokens >= 0.  Out: *pad_len.  Errors: CP_ERR_ARG.
 */
cp_status cp_ring_pad_len(int32_t cp_size, const int64_t *cached_per_rank, int64_t new_tokens,
                          int64_t *pad_len);

/*
 * Arguments of cp_attn_fwd.
 *
 * Tensors are row-major with the head dim contiguous:
 *   q  [num_q_rows][hq][dqk]    element (r,h,d) at q[r*q_row_stride + h*q_head_stride + d]
 *   k  [num_kv_rows][hkv][dqk]
 *   v  [num_kv_rows][hkv][dv]   may alias k (MLA latent: V = first dv columns of K)
 *   o  [num_q_rows][hq][dv]     dtype o_dtype
 *   lse [num_q_rows][hq]        fp32, natural log, element (r,h) at lse[r*lse_row_stride + h]
 * Strides are in elements.  q, k, v and o must be 16-byte aligned and their
 * strides multiples of 8 elements (bf16) / 4 elements (fp32).
 *
 * For row i of a segment, query head h (KV head h / (hq/hkv)), the visible
 * keys are the KV rows j in [kv_begin, kv_end) with key position
 * kpos(j) <= pos_begin + (i - q_begin) * pos_stride when causal != 0 (all of
 * them when causal == 0).  kpos(j) = kv_pos[j] when kv_pos is non-NULL,
 * else j - kv_begin.  With s_j = scale * <q, k_j>:
 *   lse = ln sum_j exp(s_j),   o = sum_j exp(s_j - lse) v_j.
 * A row with no visible key gets o = 0 and lse = -inf.
 * Rows not covered by any segment are not written.
 *
 * Paged KV (block_table != NULL; the MLA-absorbed decode shape): k and v
 * address a pool of num_kv_rows rows in blocks of block_size rows, and a
 * segment's kv range [kv_begin, kv_end) counts logical rows of request
 * seg.req: logical row x is pool row
 *   block_table[req * block_table_stride + x / block_size] * block_size
 *   + x % block_size.
 * kv_pos (if given) is indexed by logical row, per request:
 * kv_pos[req * block_table_stride * block_size + x].  Block ids outside the
 * pool are clamped into it (wrong values, never an out-of-bounds read).
 * Requirements: block_size a multiple of 32, block_table_stride >= 1,
 * num_kv_rows >= block_size (the pool holds num_kv_rows / block_size
 * blocks), every segment with req >= 0, kv_begin a multiple of 32 and
 * kv_end <= block_table_stride * block_size.
 * This is how a decode rank stores its shard when the cache is interleaved
 * over ranks in blocks ("What is Context Parallelism", section 2.2: token
 * blocks, not single tokens, on shard (i / block) mod W).
 *
 * accumulate = 1 (the pass-Q running accumulator, same blog section 3.3 and
 * the merge of section 3.6 fused into the epilogue): o and lse already hold
 * a running result (O_acc, L_acc) of the same rows; each row's new partial
 * (O_new, L_new) over this call's keys is merged into it -- m = max(L_acc,
 * L_new), w = exp(L - m), O = (w_acc O_acc + w_new O_new) / (w_acc + w_new),
 * L = m + ln(w_acc + w_new) -- and written back.  A row whose new partial is
 * empty (no visible key) is left untouched; L_acc = -inf marks an empty
 * accumulator row (its O_acc is not read), so a sequence of calls starts
 * from lse = -inf or from a first call with accumulate = 0.
 *
 * Preconditions the library cannot check (violations give unspecified
 * values, never an out-of-bounds access): each row is in at most one
 * segment; kv_pos is strictly increasing over every segment's kv range.
 *
 * segs is a HOST array (the planner's output); kv_pos is a DEVICE array
 * (int32, num_kv_rows entries; paged KV: see above) or NULL.  workspace is device memory of at
 * least cp_attn_workspace_size bytes (NULL if that size is 0).
 *
 * Supported: dtype CP_BF16 with (dqk, dv) in {(64,64), (128,128), (192,128)}
 * (needs a small workspace, see cp_attn_workspace_size); dtype CP_BF16 with
 * (dqk, dv) = (576, 512), the MLA-absorbed latent, where v must equal k with
 * equal strides (V is the first 512 columns of each latent row) -- this path
 * splits each row's keys into slices and needs a workspace; dtype CP_F32
 * with dqk = dv in {64, 128}.  o_dtype CP_BF16 or CP_F32; hq % hkv == 0;
 * scale > 0 and finite.
 */
typedef struct {
  int32_t dtype;        /* cp_dtype of q, k, v */
  int32_t o_dtype;      /* cp_dtype of o */
  int32_t num_q_rows;
  int32_t num_kv_rows;
  int32_t hq, hkv, dqk, dv;
  float scale;
  int32_t causal;
  const void *q; int64_t q_row_stride, q_head_stride;
  const void *k; int64_t k_row_stride, k_head_stride;
  const void *v; int64_t v_row_stride, v_head_stride;
  void *o;       int64_t o_row_stride, o_head_stride;
  float *lse;    int64_t lse_row_stride;
  const cp_segment *segs;  /* host */
  int32_t num_segs;
  const int32_t *kv_pos;   /* device, optional */
  void *workspace;         /* device, optional */
  size_t workspace_bytes;
  int32_t accumulate;      /* 0: write (O, LSE); 1: merge into the (O, LSE) in o / lse */
  const int32_t *block_table;  /* device, optional: paged KV (MLA decode shape only) */
  int32_t block_table_stride;  /* entries per request row of block_table */
  int32_t block_size;          /* KV rows per block (a multiple of 32) */
} cp_attn_args;

/*
 * cp_attn_workspace_size -- bytes of device workspace cp_attn_fwd needs for
 * these arguments.  bf16 (dqk, dv) in {(64,64), (128,128), (192,128)}: one
 * int32 per workgroup, i.e. 4 bytes per head per 128 or 256 query rows of
 * each segment (the kernel flags there the rare workgroups whose scores
 * outgrow the softmax reference of their first tile, and recomputes them).
 * A call too small to fill the GPU (fewer than 512 workgroups of 128 rows;
 * accumulate = 0, dense o and lse rows, no block table) cuts its long key
 * ranges into chunks and merges the chunks' partials by log-sum-exp (blog
 * section 3.6): then the workspace also holds up to 16 partial (O, LSE) per
 * row and head, in o_dtype.  The MLA-absorbed decode shape: its split-KV
 * partials; fp32: 0.  Only the shape fields, the strides, accumulate,
 * block_table and segs are read.  The contents need no initialisation and
 * are scratch after the call.
 * Errors: as cp_attn_fwd's argument checks.
 */
cp_status cp_attn_workspace_size(const cp_attn_args *args, size_t *bytes);

/*
 * cp_attn_fwd -- enqueue the attention described by `args` on `stream`.
 * Errors: CP_ERR_ARG (NULL pointers, hq % hkv != 0, a segment outside
 * [0, num_q_rows) or [0, num_kv_rows) (paged KV: outside the request's
 * logical rows), negative sizes, pos_stride < 0, positions outside
 * [-2^29, 2^30), accumulate not 0 or 1, scale not positive and finite,
 * misaligned pointers/strides, paged-KV requirements above not met),
 * CP_ERR_UNSUPPORTED (dtype or head dims without a kernel, a block table
 * with another shape than the MLA decode one, byte offsets of a tile or a
 * decode segment beyond 32 bits), CP_ERR_SMALL_BUFFER (workspace too small
 * or NULL when needed), CP_ERR_DEVICE (launch failed).
 */
cp_status cp_attn_fwd(const cp_attn_args *args, void *stream);

/*
 * cp_attn_fwd_noalloc -- cp_attn_fwd for callers that cannot allocate device
 * memory or hand over a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, same
 * kernels, same results as cp_attn_fwd, except that args->workspace and
 * args->workspace_bytes are ignored: the scratch cp_attn_workspace_size
 * would report comes instead from a static device array inside the library,
 * CP_NOALLOC_SCRATCH_BYTES bytes per GPU (placed when the library's code is
 * loaded on that GPU, held until the process ends).  The call allocates no
 * device memory (no hipMalloc / hipFree, no allocating library routine).
 * Every call on one GPU shares that GPU's array and nothing in it needs to
 * start at zero; two calls that overlap in time on the same GPU (other
 * streams, other threads) race on it and give unspecified results: order
 * them, e.g. on one stream.  Inputs and outputs are still the caller's.
 * Errors: as cp_attn_fwd; CP_ERR_SMALL_BUFFER when the call needs more than
 * CP_NOALLOC_SCRATCH_BYTES of scratch (cp_last_error then names both sizes;
 * nothing is enqueued).  The first call on a GPU looks up that GPU's array
 * address (hipGetSymbolAddress) with that GPU current; a failure there is
 * CP_ERR_DEVICE.
 */
#define CP_NOALLOC_SCRATCH_BYTES (128u << 20)
cp_status cp_attn_fwd_noalloc(const cp_attn_args *args, void *stream);

/*
 * cp_lse_merge -- merge num_parts partial results of the same rows
 * ("What is Context Parallelism", section 3.6, read as the generalised
 * online softmax): per (row, head), with m = max_j L_j,
 *   L = m + ln sum_j exp(L_j - m),   O = sum_j exp(L_j - L) O_j.
 * Partials with L_j = -inf contribute nothing and their O_j is not read; if
 * every partial is empty, O = 0 and L = -inf.
 *
 * o_parts: device, num_parts blocks of [rows][heads][dv] (contiguous, dtype
 *   part_dtype), block j starting at element j * o_part_stride.
 * lse_parts: device fp32, num_parts blocks of [rows][heads], block j at
 *   element j * lse_part_stride.
 * o_out: device [rows][heads][dv] of out_dtype; lse_out: device fp32
 *   [rows][heads] or NULL.  Outputs must not overlap the inputs.
 * Errors: CP_ERR_ARG (num_parts < 1, negative sizes, NULL pointers, strides
 *   smaller than a block, misaligned pointers, dv not a multiple of 8 or
 *   dv / 8 not a power of two up to 256),
 *   CP_ERR_UNSUPPORTED (a dtype other than CP_F32/CP_BF16), CP_ERR_DEVICE.
 */
cp_status cp_lse_merge(int32_t num_parts, int32_t rows, int32_t heads,
                       int32_t dv, const void *o_parts, int32_t part_dtype,
                       int64_t o_part_stride, const float *lse_parts,
                       int64_t lse_part_stride, void *o_out, int32_t out_dtype,
                       float *lse_out, void *stream);

/*
 * cp_calib_mfma -- sustained matrix-core rate of this GPU (a measurement
 * aid, not part of the attention path).  Each of `workgroups` workgroups of
 * 256 threads runs, per wave, `iters` rounds of 8 independent bf16 32x32x16
 * products with fp32 accumulation on register operands: 2 * 32 * 32 * 16 *
 * 8 * iters FLOPs per wave.  out: device fp32 [workgroups * 4], one value
 * per wave, 8 * 16 * iters exactly.  Errors: CP_ERR_ARG (workgroups < 1,
 * iters outside 1 .. 2^17, NULL out), CP_ERR_DEVICE.  Enqueued on `stream`.
 *
 * cp_calib_copy -- device copy dst[0, bytes) = src[0, bytes) in 16-byte
 * units, streamed past the caches (the measured copy bandwidth of this GPU:
 * bytes read + bytes written per second).  Both pointers device memory,
 * 16-byte aligned, not overlapping; bytes a multiple of 16.  Errors:
 * CP_ERR_ARG, CP_ERR_UNSUPPORTED (more than 2 TiB), CP_ERR_DEVICE.
 *
 * Both report what this chip reaches at the clock it holds under load, so
 * that kernels can be stated against a measured ceiling beside the
 * published peaks.
 */
cp_status cp_calib_mfma(int32_t workgroups, int32_t iters, float *out, void *stream);
cp_status cp_calib_copy(const void *src, void *dst, int64_t bytes, void *stream);

/* Human-readable name of a status code (static storage). */
const char *cp_status_str(int32_t status);

/* Name and description of the HIP error behind the calling thread's most
 * recent CP_ERR_DEVICE, or the sizes behind a CP_ERR_SMALL_BUFFER of
 * cp_attn_fwd_noalloc ("" if none yet).  Thread-local static storage, valid
 * until the thread's next failing call. */
const char *cp_last_error(void);

/* Library version, "major.minor.patch" (static storage). */
const char *cp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
