/*
 * seg_attn.h — C ABI of the MI355X (gfx950) segment-attention library (libsegattn.so).
 *
 * The operation is GQA attention, softmax(scale * Q K^T + mask) V, evaluated with an online
 * softmax, where each request's keys and values are not a dense tensor but a few contiguous
 * runs ("segments") of a shared token pool. This is the SegmentAttention kernel of the Flood
 * inference framework (Flood README, "Introduction": the KV cache is managed as segmentable
 * blocks instead of paged blocks, which keeps each request's cache contiguous; "Kernels /
 * Seg-attn": 64 query heads, 8 kv heads, head dim 128, measured against flash-attn's varlen
 * forward). Two entry points cover the hot path: a varlen prefill (whole or chunked, causal or
 * not) and a single-token decode that splits each request's keys into blocks, computes partial
 * results per block and reduces them per request with a log-sum-exp merge (FlashAccel article,
 * "data layout": blockwise partial attention reduced per request; the running max m_i and
 * normaliser l_i of "FlashAttention on Ascend NPU", bottleneck 2). A third writes new tokens
 * into the segments (bf16, or FP8 / INT8 quantised on write) ahead of either, and a host-side
 * allocator hands out the segments and writes the tables.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers:   every array argument is a DEVICE pointer unless marked HOST. All buffers are
 *             owned by the caller; the library never allocates, frees or retains them.
 * Streams:    work is enqueued on `stream` (0 = the null stream) and the call returns without
 *             waiting. Device-side faults surface at the caller's next synchronisation.
 * Errors:     every call returns a seg_attn_status_t. Argument errors the host can see are
 *             reported before anything is launched; nothing is printed and no C++ exception
 *             crosses the ABI. The device-resident tables (segments, cu_seqlens) are trusted on
 *             the hot path: check them with seg_attn_validate_tables on host copies if needed.
 * Layouts:    q / out          [total_q, Hq, D]   bf16, row-major, contiguous
 *             k_pool / v_pool  [pool_tokens, Hkv, D] bf16, fp8 (OCP E4M3FN) or int8,
 *                              contiguous: each (token, kv head) row is D contiguous elements
 *             k_scale/v_scale  [pool_tokens, Hkv]  fp32, FP8 and INT8 pools only: a stored
 *                              code c at (token, head) means c * scale[token, head]
 *             lse              [total_q, Hq] fp32, natural log; -inf for a row with no key
 *             segs             [nseg] seg_attn_segment_t; request b owns
 *                              segs[seg_indptr[b] .. seg_indptr[b+1]) and its logical keys are
 *                              those segments concatenated in table order
 *             cu_seqlens_q/k   [B+1] int32 prefix sums: request b has
 *                              Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] queries and
 *                              K_b = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys; K_b must equal
 *                              the sum of its segments' lengths
 * Heads:      query head h reads kv head h / (Hq / Hkv) (consecutive query heads share one).
 * Causal:     aligned bottom-right: query i of request b sits at key position K_b - Lq_b + i
 *             and sees keys 0 .. K_b - Lq_b + i (this is what chunked prefill needs).
 * Supported:  head_dim == 128 and Hq / Hkv == 8 (64 q / 8 kv heads, or any Hkv with 8 query
 *             heads per kv head; the append needs only head_dim == 128); other shapes return
 *             SEG_ATTN_ERR_UNSUPPORTED.
 */
#ifndef SEG_ATTN_H_
#define SEG_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* seg_attn_stream_t; /* a hipStream_t */

/* One contiguous run of a request's keys: pool slots [pool_offset, pool_offset + length). */
typedef struct {
  int32_t pool_offset;
  int32_t length;
} seg_attn_segment_t;

typedef int32_t seg_attn_status_t;
enum {
  SEG_ATTN_OK = 0,
  SEG_ATTN_ERR_INVALID_ARG = 1, /* a null pointer, negative size, inconsistent scalar */
  SEG_ATTN_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim != 128 or Hq/Hkv != 8 */
  SEG_ATTN_ERR_WORKSPACE = 3,   /* decode workspace missing or smaller than required */
  SEG_ATTN_ERR_HIP = 4,         /* the HIP runtime reported an error at launch */
  SEG_ATTN_ERR_TABLE = 5,       /* inconsistent tables (seg_attn_validate_tables, debug builds) */
  SEG_ATTN_ERR_OUT_OF_MEMORY = 6, /* the allocator's pool (or the host heap) cannot hold it */
  SEG_ATTN_ERR_SCRATCH = 7        /* seg_attn_decode_noalloc: more than its fixed scratch holds */
};

/* KV pool formats. FP8 and INT8 pools hold one-byte codes plus one fp32 scale per (token, kv
 * head) row; a code c at (token, head) means c * scale[token, head]. INT8 codes are two's
 * complement (the INT8 KV cache of "FlashAttention on Ascend NPU", optimisation 3). */
enum { SEG_ATTN_KV_BF16 = 0, SEG_ATTN_KV_FP8_E4M3 = 1, SEG_ATTN_KV_INT8 = 2 };

/*
 * Prefill: attention of a batch of query chunks against their requests' segmented KV.
 *
 * q            [total_q, Hq, 128] bf16, total_q = cu_seqlens_q[batch].
 * k_pool/v_pool[pool_tokens, Hkv, 128] bf16.
 * segs, seg_indptr, cu_seqlens_q, cu_seqlens_k: as in the header comment (device).
 * max_seqlen_q: HOST upper bound of every Lq_b; it sizes the launch grid. Query rows at
 *              positions >= the grid's coverage (ceil(max_seqlen_q / tile) * tile, tile 16 or 32)
 *              of a request that breaks the bound are not computed: they and their LSE are
 *              written as NaN, so the broken bound shows in the output.
 * max_seqlen_k: HOST upper bound of every K_b; with causal, max_seqlen_q <= max_seqlen_k is
 *              required (INVALID_ARG otherwise). The kernels do not depend on it otherwise.
 * softmax_scale: multiplies Q K^T (1/sqrt(128) for the usual scaling); finite and > 0
 *              (INVALID_ARG otherwise: masked keys are carried as -inf scores).
 * causal:      0 or 1. With causal and Lq_b > K_b the first Lq_b - K_b rows of request b see no
 *              key (seg_attn_validate_tables reports such tables).
 * out          [total_q, Hq, 128] bf16, written for every query row of every request; a row
 *              that sees no key gets 0 (and LSE -inf).
 * lse          [total_q, Hq] fp32 or NULL.
 * Alignment:   q, k_pool, v_pool and out 16 bytes; segs 8; the tables and lse 4
 *              (SEG_ATTN_ERR_INVALID_ARG otherwise); torch and hipMalloc allocations are.
 * Returns SEG_ATTN_OK, or an error before anything is launched.
 */
seg_attn_status_t seg_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                                   const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                   int64_t pool_tokens, float softmax_scale, int32_t causal,
                                   void* out, float* lse, seg_attn_stream_t stream);

/*
 * Decode: one query token per request (Q_len = 1) against all K_b keys of its segments.
 *
 * q            [batch, Hq, 128] bf16.
 * k_pool/v_pool[pool_tokens, Hkv, 128]: bf16 when kv_dtype == SEG_ATTN_KV_BF16, E4M3FN codes
 *              when SEG_ATTN_KV_FP8_E4M3, int8 codes when SEG_ATTN_KV_INT8 (1 byte each).
 * k_scale/v_scale [pool_tokens, Hkv] fp32 for FP8 and INT8 (required), ignored (may be NULL)
 *              for bf16. Codes are converted to bf16 exactly; k_scale multiplies the fp32
 *              scores and v_scale the fp32 probabilities before their bf16 rounding.
 * softmax_scale: as for seg_attn_prefill (finite and > 0).
 * cu_seqlens_k [batch+1] int32; max_seqlen_k: HOST upper bound of every K_b; it sizes the
 *              workspace. If some K_b exceeds it, nothing is computed and every output and
 *              LSE of the call is written as NaN, so the broken bound shows in the output.
 * num_splits   0: each request's keys are cut into chunks whose length the device picks from the
 *              total key count (at least 512 keys for bf16, 1024 for fp8 / int8) so that every compute
 *              unit gets several (chunk, kv head) work units. n > 0: chunks of
 *              ceil(max_seqlen_k / n) keys rounded up to a multiple of 64, so at most n per
 *              request. A request cut into one chunk is written directly; otherwise each chunk's
 *              partial (O_s, LSE_s) goes to the workspace and a merge kernel combines them.
 *              The chunks are listed on the device: by the split workgroups themselves when
 *              num_splits = 0 and batch <= 256, otherwise by a one-workgroup plan kernel
 *              launched first. Both list the same chunks, so the results are the same bit for
 *              bit; the environment variable SEG_ATTN_DECODE_PLAN=kernel selects the plan
 *              kernel for every call.
 * out          [batch, Hq, 128] bf16; lse [batch, Hq] fp32 or NULL. A request with K_b = 0
 *              gets out = 0 and lse = -inf.
 * workspace    device scratch of at least seg_attn_decode_workspace_bytes(...) bytes for the
 *              same (batch, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, kv_dtype,
 *              num_splits); always required. It holds the chunk plan and the partial results;
 *              its contents need no initialisation and are clobbered.
 * Alignment:   q, k_pool and v_pool 16 bytes, out 8, segs 8, tables, scales and lse 4
 *              (SEG_ATTN_ERR_INVALID_ARG otherwise); workspace 16 (SEG_ATTN_ERR_WORKSPACE).
 */
seg_attn_status_t seg_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                                  const float* k_scale, const float* v_scale, int32_t kv_dtype,
                                  const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                  const int32_t* cu_seqlens_k, int32_t batch,
                                  int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv,
                                  int32_t head_dim, int64_t pool_tokens, float softmax_scale,
                                  int32_t num_splits, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, seg_attn_stream_t stream);

/*
 * Decode without any allocation, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The same computation and
 * arguments as seg_attn_decode without the workspace: the plan and partial results live in a
 * fixed scratch array of 64 MiB that the library keeps on every GPU it runs on until the process
 * ends (its address is looked up on the first call on a device). The call allocates nothing.
 * With num_splits = 0 the plan needs at most (6 * max(1, CUs / Hkv) + 2 * batch) chunks, with
 * num_splits = n at most n * batch; each chunk takes Hq * 129 * 4 + 64 bytes (33 088 for
 * Hq = 64), so 64 MiB holds about 2000 chunks (batch <= about 900 at Hq = 64 with automatic
 * splits). A call that needs more returns SEG_ATTN_ERR_SCRATCH before anything is launched.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU (on
 * different streams, or from several host threads) race and must be serialised by the caller.
 * Every part of the scratch a call reads is written earlier in the same call.
 */
seg_attn_status_t seg_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                          const float* k_scale, const float* v_scale,
                                          int32_t kv_dtype, const seg_attn_segment_t* segs,
                                          const int32_t* seg_indptr, const int32_t* cu_seqlens_k,
                                          int32_t batch, int32_t max_seqlen_k, int32_t num_heads_q,
                                          int32_t num_heads_kv, int32_t head_dim,
                                          int64_t pool_tokens, float softmax_scale,
                                          int32_t num_splits, void* out, float* lse,
                                          seg_attn_stream_t stream);

/* Bytes of workspace seg_attn_decode needs for these arguments: a 256-byte plan header, the
 * per-request chunk offsets, a 64-byte record per chunk and one fp32 (O, LSE) partial per chunk and query
 * head, for the largest chunk count the arguments allow. Returns 0 for invalid or unsupported
 * sizes; seg_attn_decode reports those. */
size_t seg_attn_decode_workspace_bytes(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_q,
                                       int32_t num_heads_kv, int32_t head_dim, int32_t kv_dtype,
                                       int32_t num_splits);

/* The largest number of chunks seg_attn_decode cuts one request into for these arguments (at
 * least 1). Writes the chunk length to *split_len when it is not NULL: the fixed length for
 * num_splits > 0, the smallest length the device may pick for 0. Returns -1 on invalid sizes. */
int32_t seg_attn_decode_num_splits(int32_t batch, int32_t max_seqlen_k, int32_t num_heads_kv,
                                   int32_t kv_dtype, int32_t num_splits, int32_t* split_len);

/*
 * KV append: write a batch's new tokens' K and V rows into the pool slots their requests'
 * segments give them, the step that precedes attention on every prefill chunk and decode token.
 * The pages imply it without describing it: each request's cache is a few contiguous segments
 * of one shared pool (Flood README, "Introduction"), and an FP8 KV cache is among the same
 * README's features; the FP8 row format is the one seg_attn_decode reads.
 *
 * k_new/v_new  [total_new, Hkv, 128] bf16, the new tokens of all requests in request order.
 * segs, seg_indptr: the tables AFTER the caller has grown each request's segments to hold its
 *              new tokens (device).
 * cu_seqlens_new [batch+1] int32 (device): request b appends
 *              n_b = cu_seqlens_new[b+1] - cu_seqlens_new[b] tokens, rows
 *              cu_seqlens_new[b] .. cu_seqlens_new[b+1]-1 of k_new/v_new.
 * cu_seqlens_k [batch+1] int32 (device): key counts K_b AFTER the append. Request b's new
 *              tokens become its last n_b keys, logical positions K_b - n_b .. K_b - 1, in row
 *              order; n_b <= K_b and the segment lengths of b must sum to K_b.
 * total_new    HOST, must equal cu_seqlens_new[batch]; it sizes the launch.
 * kv_dtype     SEG_ATTN_KV_BF16: rows are copied bit for bit. SEG_ATTN_KV_FP8_E4M3: per
 *              (token, kv head) row x the scale s = max|x| / 448 in fp32 (1 for an all-zero row)
 *              goes to k_scale/v_scale[slot, head] and the codes E4M3FN(clamp(x / s, +-448)),
 *              x / s an fp32 division and the conversion rounding to nearest, ties to even, go
 *              to the pool; the largest |x| of a row is stored as +-448. SEG_ATTN_KV_INT8: the
 *              same with s = max|x| / 127 and codes round-half-even(clamp(x / s, +-127)) as
 *              two's-complement bytes (-128 is never written).
 *              New rows must be finite.
 * k_pool/v_pool[pool_tokens, Hkv, 128] bf16, E4M3FN or int8 bytes; k_scale/v_scale
 *              [pool_tokens, Hkv] fp32 for FP8 and INT8 (required), ignored for bf16. Only the new tokens' slots (and their
 *              scales) are written; every other slot is left as it was.
 * k_new, v_new and bf16 pools must be 16-byte aligned, FP8 / INT8 pools 8-byte, scales 4-byte
 * (SEG_ATTN_ERR_INVALID_ARG otherwise); torch and hipMalloc allocations are.
 * A key whose slot falls outside the request's segments or the pool is skipped, never written
 * out of bounds; this only happens with tables that break the rules above. New tokens of
 * different requests must not share a slot (the writes would race).
 * Returns SEG_ATTN_OK, or an error before anything is launched.
 */
seg_attn_status_t seg_attn_kv_append(const void* k_new, const void* v_new,
                                     const seg_attn_segment_t* segs, const int32_t* seg_indptr,
                                     const int32_t* cu_seqlens_new, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_new, int32_t num_heads_kv,
                                     int32_t head_dim, int64_t pool_tokens, int32_t kv_dtype,
                                     void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                     seg_attn_stream_t stream);

/*
 * Segment linear attention: simple gated linear attention over a pool of per-request states, the
 * kernel family of the Flood README's "Seg-linear-attn" table (16 heads, 16 kv heads, head dim
 * 128, against flash-linear-attention's chunked and recurrent simple GLA). Per request and head,
 * with a log decay g_t <= 0 per token and head:
 *   S_t = exp(g_t) S_{t-1} + k_t^T v_t,   o_t = scale * q_t S_t   (S: 128 x 128)
 * q, k, v      [T, H, 128] bf16 (query and kv heads are equal in number); g [T, H] fp32.
 * state_pool   [pool_slots, H, 128, 128] fp32: request b's state is slot state_slots[b] (rows
 *              are d_k, the 128 d_v values of a row contiguous). Slots must be distinct within a
 *              call; a slot outside [0, pool_slots) makes its request a no-op.
 * out          [T, H, 128] bf16.
 * Prefill: request b's tokens are rows cu_seqlens[b] .. cu_seqlens[b+1]-1; its state starts
 * from its slot (initial_state = 1) or from zero (0) and the final state is written back to the
 * slot. The products run on bf16 operands with fp32 accumulation and an fp32 state. Three
 * evaluation orders of the same recurrence:
 *   - workspace != NULL and max_seqlen <= 4096: one launch of the closed form
 *     o_t = scale (exp(G_t) q_t S_0 + sum_{s<=t} (q_t . k_s) exp(G_t - G_s) v_s), G the running
 *     sum of g, with the final state from the same sums; the workspace is not used (a stored
 *     initial state takes a second launch, for the states, after the outputs have read S_0);
 *   - workspace != NULL and longer requests: 64-token chunks of all requests in parallel, with a
 *     scan carrying the state between them; the workspace must hold
 *     seg_attn_linear_prefill_workspace_bytes(batch, max_seqlen, H, 128) bytes, 256-byte aligned
 *     (contents clobbered); the environment variable SEG_ATTN_LINEAR_PREFILL=chunked selects this
 *     order at every length;
 *   - workspace = NULL: one workgroup per (request, head, half of d_v) walks the request's
 *     64-token chunks in order; max_seqlen is unused.
 * With a workspace, max_seqlen (HOST) must be at least every request's length: a longer request
 * is not processed past it (rounded up to 64 tokens), and its later tokens' outputs and its
 * final state are written as NaN so the broken bound shows.
 * Decode: one token per request (row b), state read from and written to the slot, in fp32
 * throughout. Buffers: q, k, v and the pool 16-byte aligned, out 8-byte.
 * Returns SEG_ATTN_OK, or an error before anything is launched.
 */
seg_attn_status_t seg_attn_linear_prefill(const void* q, const void* k, const void* v,
                                          const float* g, const int32_t* cu_seqlens,
                                          const int32_t* state_slots, int32_t batch,
                                          int32_t max_seqlen, int32_t num_heads, int32_t head_dim,
                                          float scale, int32_t initial_state, float* state_pool,
                                          int64_t pool_slots, void* out, void* workspace,
                                          size_t workspace_bytes, seg_attn_stream_t stream);
/* Workspace bytes of the chunk-parallel linear prefill (0 for invalid or unsupported sizes). */
size_t seg_attn_linear_prefill_workspace_bytes(int32_t batch, int32_t max_seqlen, int32_t num_heads,
                                               int32_t head_dim);
seg_attn_status_t seg_attn_linear_decode(const void* q, const void* k, const void* v, const float* g,
                                         const int32_t* state_slots, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, float scale,
                                         float* state_pool, int64_t pool_slots, void* out,
                                         seg_attn_stream_t stream);

/*
 * Segment allocator (host only; no GPU call). Hands out ranges of a pool of `pool_tokens` slots
 * to requests, keeping each request's cache in as few contiguous segments as the free space
 * allows (Flood README, "Introduction": segmentable blocks instead of paged blocks, for the
 * continuity of each request's cache), and writes the tables the entry points above take.
 *
 * Policy: a request owns slot ranges holding C slots (its capacity), in the order they were
 * added; its L <= C keys are the first L of them, and the tables list only those. Growing a
 * request by n keys uses spare capacity first; a shortfall of m slots is allocated aiming at
 * m rounded up to the allocator's granule (exactly m if that does not fit), so that a request
 * growing one token at a time gets a new range only every `granule` tokens; reserve sets
 * capacity aside for a known final length. An allocation first extends the request's last
 * range over the free slots that directly follow it; the rest goes to the smallest free run
 * that holds it (lowest start among equals), from the run's start; if no run holds it, the
 * largest run (lowest start among equals) gives what it has and the rest is placed the same
 * way. Released and truncated slots merge with neighbouring free runs.
 *
 * Requests are named by any int64 id; an id never grown has no keys. The allocator tracks slots
 * only: moving K/V data is the caller's (seg_attn_kv_append writes new tokens). One allocator
 * must not be used from two threads at once. A SEG_ATTN_ERR_OUT_OF_MEMORY caused by the pool
 * (n larger than the free slots) changes nothing; one caused by a failing host allocation
 * leaves the allocator unusable (destroy it).
 */
typedef struct seg_attn_allocator seg_attn_allocator_t;

/* A new allocator over slots [0, pool_tokens), all free; pool_tokens <= INT32_MAX; growth
 * shortfalls are rounded up to `granule` >= 1 slots (1: exact). */
seg_attn_status_t seg_attn_allocator_create(int64_t pool_tokens, int64_t granule,
                                            seg_attn_allocator_t** out);
void seg_attn_allocator_destroy(seg_attn_allocator_t* allocator);

/* Add n >= 0 keys to `request` (as above). SEG_ATTN_ERR_OUT_OF_MEMORY, with nothing changed,
 * if its spare capacity and the free slots together hold fewer than n. */
seg_attn_status_t seg_attn_allocator_grow(seg_attn_allocator_t* allocator, int64_t request,
                                          int64_t n);
/* seg_attn_allocator_grow(requests[i], n[i]) for i = 0 .. count-1 in order, stopping at the
 * first that fails (whose status is returned); *done (if not NULL) receives how many were
 * applied. One call per decode step instead of one per request. */
seg_attn_status_t seg_attn_allocator_grow_batch(seg_attn_allocator_t* allocator,
                                                const int64_t* requests, const int64_t* n,
                                                int32_t count, int32_t* done);
/* Make the capacity of `request` at least `capacity` slots without adding keys (a no-op if it is
 * already); SEG_ATTN_ERR_OUT_OF_MEMORY, with nothing changed, if the free slots do not hold the
 * difference. */
seg_attn_status_t seg_attn_allocator_reserve(seg_attn_allocator_t* allocator, int64_t request,
                                             int64_t capacity);
/* Free every slot of `request` and forget it (a no-op for an unknown id). */
seg_attn_status_t seg_attn_allocator_release(seg_attn_allocator_t* allocator, int64_t request);
/* Keep the first new_length keys of `request` and free every later slot it owns, spare capacity
 * included (a no-op if it has no more than new_length keys). */
seg_attn_status_t seg_attn_allocator_truncate(seg_attn_allocator_t* allocator, int64_t request,
                                              int64_t new_length);
/* Keys (length) and owned slots (capacity) of `request` (0 if unknown), or -1 for a NULL
 * allocator. */
int64_t seg_attn_allocator_length(const seg_attn_allocator_t* allocator, int64_t request);
int64_t seg_attn_allocator_capacity(const seg_attn_allocator_t* allocator, int64_t request);

/*
 * HOST tables for the batch requests[0 .. batch): segs [*nseg] (capacity segs_capacity),
 * seg_indptr [batch+1] and cu_seqlens_k [batch+1], in the layout of the header comment, ready to
 * be copied to the device. *nseg (if not NULL) receives the number of segments needed; when it
 * exceeds segs_capacity nothing else is written and SEG_ATTN_ERR_WORKSPACE is returned.
 */
seg_attn_status_t seg_attn_allocator_tables(const seg_attn_allocator_t* allocator,
                                            const int64_t* requests, int32_t batch,
                                            seg_attn_segment_t* segs, int64_t segs_capacity,
                                            int32_t* seg_indptr, int32_t* cu_seqlens_k,
                                            int64_t* nseg);

/*
 * Compaction: relocate fragmented requests so that each becomes one contiguous range, the
 * continuity the Flood README ("Introduction") keeps each request's cache in segmentable blocks
 * for. Requests owning two or more ranges are taken in order of decreasing range count, then
 * increasing id; each moves whole (its capacity C) into the smallest free run that existed when
 * the call began and still holds C (lowest start among equals), from the run's start; a request
 * that fits nowhere stays as it is. Slots the call frees are not reused within it, so every
 * destination is disjoint from every source and from every other destination.
 *
 * The allocator's state (tables, free runs) is updated at once; the pool data must then be moved
 * with seg_attn_kv_move (HOST moves copied to the device) before the new tables are used and
 * before any further append. moves [capacity] receives one record per key-holding range of a
 * relocated request: copy `length` slots from src_offset to dst_offset; `first` is the number of
 * slots of all earlier records. *n_moves (if not NULL) receives the number of records; when it
 * exceeds capacity nothing changes and SEG_ATTN_ERR_WORKSPACE is returned.
 */
typedef struct {
  int32_t src_offset;
  int32_t dst_offset;
  int32_t length;
  int32_t first;
} seg_attn_move_t;
seg_attn_status_t seg_attn_allocator_compact(seg_attn_allocator_t* allocator, seg_attn_move_t* moves,
                                             int64_t capacity, int64_t* n_moves);

/*
 * KV move: apply a move list (from seg_attn_allocator_compact) to the pools on the device. For
 * each record, the rows of slots src_offset .. src_offset + length - 1 (every kv head; K, V and,
 * for FP8 / INT8 pools, their scales) are copied to the slots from dst_offset. The records'
 * sources and destinations must be pairwise disjoint (the allocator plans them so); rows are
 * copied in parallel, in no particular order.
 * moves        [n_moves] seg_attn_move_t, DEVICE, 16-byte aligned; `first` must be the running
 *              sum of the earlier records' lengths.
 * total_tokens HOST, the sum of all lengths (it sizes the launch); at most pool_tokens.
 * k_pool/v_pool/k_scale/v_scale as for seg_attn_kv_append (bf16 pools 16-byte aligned, one-byte
 *              pools 8-byte, scales 4-byte; scales ignored for bf16).
 * A slot outside [0, pool_tokens) is skipped, never accessed.
 * Returns SEG_ATTN_OK, or an error before anything is launched.
 */
seg_attn_status_t seg_attn_kv_move(const seg_attn_move_t* moves, int32_t n_moves,
                                   int64_t total_tokens, int32_t num_heads_kv, int32_t head_dim,
                                   int64_t pool_tokens, int32_t kv_dtype, void* k_pool,
                                   void* v_pool, float* k_scale, float* v_scale,
                                   seg_attn_stream_t stream);

/* Free slot count, longest free run, number of free runs and of live requests (any may be NULL). */
seg_attn_status_t seg_attn_allocator_stats(const seg_attn_allocator_t* allocator,
                                           int64_t* free_tokens, int64_t* largest_free_run,
                                           int64_t* free_runs, int64_t* requests);

/* The free runs in pool order as (start, length) pairs; *count receives their number, and if
 * it exceeds capacity nothing else is written and SEG_ATTN_ERR_WORKSPACE is returned. */
seg_attn_status_t seg_attn_allocator_free_runs(const seg_attn_allocator_t* allocator,
                                               seg_attn_segment_t* runs, int64_t capacity,
                                               int64_t* count);

/* Static text for a status code; never NULL. */
const char* seg_attn_status_string(seg_attn_status_t status);

/*
 * Check HOST copies of the tables against each other and the pool: every segment inside
 * [0, pool_tokens) with length >= 0, seg_indptr and cu_seqlens non-decreasing from 0, each
 * request's segment lengths summing to K_b, Lq_b <= K_b when causal, no two segments of the
 * whole table overlapping. cu_seqlens_q may be NULL (decode: Lq_b = 1). On failure returns
 * SEG_ATTN_ERR_TABLE and, if bad_index is not NULL, stores the offending request (or segment,
 * for overlaps and out-of-pool segments) index there.
 */
seg_attn_status_t seg_attn_validate_tables(const seg_attn_segment_t* segs, int64_t nseg,
                                           const int32_t* seg_indptr,
                                           const int32_t* cu_seqlens_q,
                                           const int32_t* cu_seqlens_k, int32_t batch,
                                           int64_t pool_tokens, int32_t causal,
                                           int64_t* bad_index);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t seg_attn_version(void);

/*
 * 1 for the library built with SEG_ATTN_DEBUG (libsegattn_debug.so, for tests and bring-up),
 * 0 for the release library. The debug build synchronises the stream before every attention
 * call (prefill and decode, including the entry point that allocates nothing), copies the segment
 * tables back to the host and checks them as seg_attn_validate_tables does, except that segments
 * of different requests may share slots (attention only reads them). Broken tables make the call
 * return SEG_ATTN_ERR_TABLE with nothing launched, so no kernel resolves a pool slot outside
 * [0, pool_tokens). The check costs a host round trip per call.
 */
int32_t seg_attn_debug_build(void);

#ifdef __cplusplus
}
#endif

#endif /* SEG_ATTN_H_ */
