/*
 * pkv.h -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.so.  Four entry points make up the decode hot path of a
 * paged KV cache:
 *
 *   kv_cache_append               write each new token's K/V into its slot
 *   paged_attention_decode        one query token per sequence, attending over
 *                                 the sequence's cached K/V reached through its
 *                                 block table, with an online softmax
 *   paged_attention_decode_split  the same over fixed-size partitions of each
 *                                 sequence's context ("flash-decoding" style
 *                                 split), writing per-partition results
 *   split_reduce                  log-sum-exp weighted merge of the partitions
 *   paged_decode_step             append + split pass + merge in one launch
 *   paged_attention_prefill       a chunk of new tokens per sequence attending
 *                                 causally over the cache (chunked prefill),
 *                                 also split over context partitions
 *
 * plus a host-side block allocator (pkv_allocator_*) that hands out the
 * cache's blocks and builds block tables and slot mappings for a batch.
 *
 * Sources (the pages describing the method):
 *   - nanoserve project write-up, section "What I built": a paged KV cache
 *     (block allocator plus per-sequence block tables) and a fused decode
 *     kernel that runs an online softmax over the block table.
 *   - the nanoserve author's post thread, Day 74 post: a split-attention
 *     ("flash-decoding style") decode arm next to the plain one.
 *   - Inference Engineering, Day 11 post (how vLLM works): every step writes
 *     the new key and value vectors into the cache, whose fixed-size blocks
 *     are handed out per request from a free-block queue on the host.
 *   - Inference Engineering, Day 12 post (chunked prefill): a long prompt is
 *     processed, and written to the cache, a chunk per pass.
 * The pages give no signatures, layouts or merge rule; the choices below are
 * this library's and are the plainest reading of the pages.
 *
 * Conventions common to every call
 * --------------------------------
 *  - fp16 means IEEE binary16 (_Float16).  Every tensor is dense, row-major,
 *    with the shape given in its comment.
 *  - Every pointer is device memory owned by the caller.  The library holds
 *    no state, never allocates, never synchronises and never reads device
 *    data on the host.  Work is enqueued on `stream` (a hipStream_t passed as
 *    void*; NULL is the null stream) and runs asynchronously.
 *  - K/V pools have the layout [num_blocks, block_size, num_kv_heads,
 *    head_dim]; one pool holds K, another V.  Logical position t of sequence
 *    b lives in physical block block_tables[b, t / block_size] at offset
 *    t % block_size.
 *  - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *  - Supported shapes: head_dim 64 or 128; block_size a multiple of 16 in
 *    [16, 256]; num_q_heads / num_kv_heads <= 16.
 *  - Alignment: fp16 and fp32 tensors 16 bytes, int32 arrays 4 bytes,
 *    slot_mapping 8 bytes.
 *  - Empty calls (num_tokens == 0, B == 0) return PKV_OK without launching;
 *    their per-token / per-sequence pointers may then be NULL.
 *  - Return value: PKV_OK, or a negative status.  PKV_ERR_INVALID_ARG and
 *    PKV_ERR_UNSUPPORTED are decided from the arguments alone, before any
 *    HIP call, and nothing is launched.  PKV_ERR_LAUNCH reports a HIP error
 *    from the launch (hipGetLastError).
 *  - Device data contract (not checkable on the host): context_lens[b] in
 *    [0, max_blocks_per_seq * block_size]; block_tables[b, i] in
 *    [0, num_blocks) for i < ceil(context_lens[b] / block_size); entries past
 *    that may be read (the whole [B, max_blocks_per_seq] array must be
 *    readable) but their values are never used.  The kernels guard themselves: a context length
 *    outside the range is clamped into it, and a block id outside
 *    [0, num_blocks) is not read and its positions do not contribute.  So a
 *    contract violation gives wrong numbers, never an out-of-bounds access.
 *  - Outputs must not alias inputs.  Calls that write the same memory race
 *    unless ordered by the stream.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment, ...   */
  PKV_ERR_UNSUPPORTED = -2, /* head_dim / block_size / group not compiled  */
  PKV_ERR_LAUNCH = -3,      /* HIP reported an error for the launch        */
  PKV_ERR_NO_SPACE = -4,    /* allocator: not enough free blocks, or a
                               sequence would pass max_blocks_per_seq      */
  PKV_ERR_SCRATCH = -5      /* paged_decode_step_noalloc: the call needs more
                               than its static scratch holds               */
};

/* Static, human-readable name of a status code. */
const char* pkv_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int pkv_version(void);

/*
 * pkv_launch_config -- an explicit launch shape for one call of an attention
 * pass, taken by the _ex entry points (paged_attention_decode_ex,
 * paged_attention_decode_split_ex, paged_decode_step_ex); the calls without
 * _ex use the defaults.  The library keeps no setting between calls.  Every
 * field 0 means the library's default.
 *   waves_per_group    wavefronts (64 lanes) per workgroup: 1, 2, 4 or 8;
 *                      they share the workgroup's context range (a whole
 *                      sequence unsplit, one partition in the split pass and
 *                      the fused step).  Defaults: 8 unsplit, 4 split; the
 *                      fused step takes 4, or 8 when the grid is at most 256
 *                      workgroups and a pair has at least 8 partitions.
 *   subtiles_per_tile  16-token subtiles a wave loads per tile: 1, 2 or 4
 *                      (defaults: 2 at head_dim 64 except the fused step's 1;
 *                      1 at head_dim 128).
 *   tiles_in_flight    tiles of K/V a wave keeps in flight: 2 or 4 (default 2).
 *   grid               split pass and fused step: 0 auto (direct up to 8192
 *                      workgroups, compact above), 1 direct (a workgroup per
 *                      sequence, KV head and group of partitions, empty ones
 *                      included), 2 compact (a fixed number of workgroups,
 *                      each scanning the context lengths and looping over the
 *                      non-empty groups; B <= 4096).  The compact grid runs
 *                      the default shape only: a call that sets another
 *                      shape is launched direct.
 * Shapes beyond the register budget (more than 8 subtiles in flight at
 * head_dim 64, 4 at head_dim 128) are reduced to fit.  Results do not
 * depend on the shape beyond fp32 summation order.  A field outside its set
 * gives PKV_ERR_INVALID_ARG.  NULL means every default.
 */
typedef struct pkv_launch_config {
  int32_t waves_per_group;
  int32_t subtiles_per_tile;
  int32_t tiles_in_flight;
  int32_t grid;
} pkv_launch_config;

/*
 * kv_cache_append -- write the K and V rows of new tokens into their slots.
 *
 * Defined by the cache update of every decode step (Inference Engineering,
 * Day 11 post) into the block layout of the nanoserve paged cache ("What I
 * built").  Also serves chunked prefill: several tokens of one sequence, in
 * any number of blocks, in one call (Inference Engineering, Day 12 post).
 *
 *   k_pool, v_pool  [num_blocks, block_size, num_kv_heads, head_dim] fp16,
 *                   updated in place.
 *   k_new, v_new    [num_tokens, num_kv_heads, head_dim] fp16.
 *   slot_mapping    [num_tokens] int64: slot = block * block_size + offset.
 *                   A negative slot, or one >= num_blocks * block_size, skips
 *                   that token.  Slots must be unique within a call.
 *
 * The copy is bit-exact.  num_tokens == 0 is a no-op that returns PKV_OK.
 */
int kv_cache_append(void* k_pool, void* v_pool,
                    const void* k_new, const void* v_new,
                    const int64_t* slot_mapping,
                    int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * paged_attention_decode -- single-token decode attention over the paged
 * cache, online softmax over the block table (nanoserve write-up, "What I
 * built", fused paged-attention decode kernel):
 *
 *   out[b, h, :] = sum_t softmax_t(scale * q[b, h, :] . K_b[t, :]) V_b[t, :]
 *
 * over t < context_lens[b], with K_b, V_b the rows of KV head
 * h / (num_q_heads / num_kv_heads) reached through block_tables[b].
 *
 *   out           [B, num_q_heads, head_dim] fp16 (written).
 *   q             [B, num_q_heads, head_dim] fp16.
 *   k_pool/v_pool [num_blocks, block_size, num_kv_heads, head_dim] fp16.
 *   block_tables  [B, max_blocks_per_seq] int32.
 *   context_lens  [B] int32, positions attended (including the token this
 *                 step appended).  0 gives an all-zero output row.
 *   scale         softmax scale (finite), applied to the fp32 dot product.
 *
 * All arithmetic is fp32 (fp16 products, fp32 accumulation); the output is
 * rounded to fp16 (nearest even).  One workgroup serves one (sequence, KV
 * head) pair, so this call fills the GPU only when B * num_kv_heads is
 * large; the split call below spreads long contexts over the whole GPU.
 * B == 0 is a no-op.
 */
int paged_attention_decode(void* out, const void* q,
                           const void* k_pool, const void* v_pool,
                           const int32_t* block_tables,
                           const int32_t* context_lens,
                           int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq,
                           float scale, void* stream);

/* paged_attention_decode with an explicit launch shape (see
 * pkv_launch_config; NULL = defaults). */
int paged_attention_decode_ex(void* out, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables,
                              const int32_t* context_lens,
                              int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              float scale, const pkv_launch_config* config,
                              void* stream);

/*
 * paged_attention_decode_split -- split-context pass of the flash-decoding
 * style arm (nanoserve author's post thread, Day 74).  Partition p of
 * sequence b covers logical positions [p * partition_size,
 * min((p + 1) * partition_size, context_lens[b])).  For every partition that
 * holds at least one position:
 *
 *   partial_out[b, h, p, :] = softmax-weighted sum of V over the partition
 *                             (normalised within the partition), fp32;
 *   partial_lse[b, h, p]    = ln(sum_t exp(scale * q . K_t)) over the
 *                             partition, fp32.
 *
 * For a partition that starts at or past context_lens[b], partial_lse is set
 * to -inf and partial_out is left untouched.
 *
 *   partial_out     [B, num_q_heads, max_partitions, head_dim] fp32 workspace.
 *   partial_lse     [B, num_q_heads, max_partitions] fp32 workspace.
 *   partition_size  a multiple of block_size.
 *   max_partitions  with max_partitions * partition_size >=
 *                   max_blocks_per_seq * block_size.
 * Other arguments as for paged_attention_decode.
 */
int paged_attention_decode_split(float* partial_out, float* partial_lse,
                                 const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables,
                                 const int32_t* context_lens,
                                 int32_t B, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq,
                                 int32_t partition_size, int32_t max_partitions,
                                 float scale, void* stream);

/* paged_attention_decode_split with an explicit launch shape (see
 * pkv_launch_config; NULL = defaults). */
int paged_attention_decode_split_ex(float* partial_out, float* partial_lse,
                                    const void* q,
                                    const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables,
                                    const int32_t* context_lens,
                                    int32_t B, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq,
                                    int32_t partition_size, int32_t max_partitions,
                                    float scale, const pkv_launch_config* config,
                                    void* stream);

/*
 * paged_decode_step -- one whole decode step in a single launch: the cache
 * write of kv_cache_append, the split pass of paged_attention_decode_split
 * and the merge of split_reduce, fused.  This is the launch-overhead remedy
 * the pages point to (nanoserve write-up, "Results": decode time is mostly
 * launch overhead; the author's post thread, Day 74: a CUDA-graphed arm).
 *
 *   out, lse_out      as split_reduce (lse_out may be NULL).
 *   k_pool, v_pool    the pools, updated in place by the append.
 *   q                 [B, num_q_heads, head_dim] fp16.
 *   k_new, v_new      [B, num_kv_heads, head_dim] fp16: one new token per
 *                     sequence.
 *   slot_mapping      [B] int64, the new token's slot, or NULL for no append
 *                     (then k_new/v_new may be NULL).  A negative slot, or one
 *                     past the pool, skips that sequence's append.  The slot
 *                     must be the one of position context_lens[b] - 1 in the
 *                     sequence's block table (the decode step's new token); the
 *                     step then attends over it exactly as append followed by
 *                     decode would.  Any other slot is still written, but
 *                     whether this step's attention sees the new value there
 *                     is undefined.
 *   partial_out       [B, num_q_heads, max_partitions, head_dim] fp32 and
 *   partial_lse       [B, num_q_heads, max_partitions] fp32 workspace, all
 *                     zero before the first call; every call leaves them so
 *                     (rows in flight are stored bit-inverted, so a zero word
 *                     means "not written").  num_q_heads / num_kv_heads *
 *                     max_partitions * head_dim * 4 must be below 2^30
 *                     (else PKV_ERR_UNSUPPORTED).  Not to be shared with
 *                     paged_attention_decode_split, which leaves values there.
 *   counters          [B, num_kv_heads, 32] int32 workspace, 8-byte aligned
 *                     (one 128-byte line per sequence and KV head, so
 *                     tickets of different pairs never contend for a line):
 *                     must be zero before the first call; every call leaves
 *                     it zero.
 * Calls that share a workspace must be ordered by a stream; a call that
 * faults or is aborted leaves it undefined (initialise it again).
 * Other arguments as for paged_attention_decode_split.
 *
 * Each (sequence, KV head) with more than one non-empty partition is merged
 * in the launch by its workgroups: each takes a ticket from the pair's
 * counter line early, and the holder of the last ticket merges, reading the
 * other partitions' rows once none of their words is zero (device-coherent
 * accesses; the others never wait).  A pair with more than 32 partitions
 * merges in two levels: the partitions form groups of about 8, the last
 * ticket of each group merges the group into its own row, and the pair's
 * last ticket merges the group results.  Mergers set the rows and words they
 * read back to zero.  Their waits are bounded in time (20 ms): a workspace that breaks
 * the contract above gives wrong numbers, not a stalled queue.  A sequence
 * that fits one partition is written directly.  Results equal append +
 * split pass + split_reduce up to fp32 summation order, and do not depend
 * on which workgroups merge.
 */
int paged_decode_step(void* out, float* lse_out,
                      void* k_pool, void* v_pool,
                      const void* q, const void* k_new, const void* v_new,
                      const int64_t* slot_mapping,
                      const int32_t* block_tables, const int32_t* context_lens,
                      float* partial_out, float* partial_lse, int32_t* counters,
                      int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                      int32_t max_blocks_per_seq, int32_t partition_size,
                      int32_t max_partitions, float scale, void* stream);

/* paged_decode_step with an explicit launch shape (see pkv_launch_config;
 * NULL = defaults). */
int paged_decode_step_ex(void* out, float* lse_out,
                         void* k_pool, void* v_pool,
                         const void* q, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float* partial_out, float* partial_lse, int32_t* counters,
                         int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t partition_size,
                         int32_t max_partitions, float scale,
                         const pkv_launch_config* config, void* stream);

/*
 * paged_decode_step_noalloc -- paged_decode_step with no workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * step's workspace (partials, their lse, ticket counters) lives in a static
 * device array of the library, 16 MiB per GPU, held by each GPU the library
 * runs on until the process ends; a call needs
 *   round256(B * num_q_heads * max_partitions * head_dim * 4)
 *   + round256(B * num_q_heads * max_partitions * 4)
 *   + round256(B * num_kv_heads * 128)
 * bytes of it (round256 = rounded up to a multiple of 256), and returns
 * PKV_ERR_SCRATCH, before any HIP call, when that is more than 16 MiB (at
 * head_dim 64 with 14 query heads: about 4,600 sequence-partitions, e.g.
 * B=32 at up to 144 partitions each).
 *
 * The call allocates nothing: no hipMalloc, hipFree or allocating library
 * routine.  Its first call on a device (the current device, which must be
 * the stream's) resolves the array's address there and clears it once with
 * a fill kernel on `stream`.  Every call on a GPU shares that GPU's array
 * and leaves it all zero, as the workspace contract of paged_decode_step
 * asks; calls that overlap on one GPU (on different streams without an
 * ordering between them, or from several host threads) race on it and give
 * undefined results, and a call that faults or is aborted leaves it
 * undefined.  Arguments, outputs, results and errors are otherwise those of
 * paged_decode_step.
 */
int paged_decode_step_noalloc(void* out, float* lse_out,
                              void* k_pool, void* v_pool,
                              const void* q, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t partition_size,
                              int32_t max_partitions, float scale, void* stream);

/*
 * paged_attention_prefill -- attention of a chunk of new tokens per sequence
 * over the paged cache (chunked prefill: Inference Engineering, Day 12 post
 * on chunked prefill in vLLM, where a long prompt is processed a chunk per
 * pass and each pass writes its K/V into the cache).  Sequence b's chunk is
 * rows query_start[b] .. query_start[b+1]-1 of q (n_b rows); it holds the last
 * n_b of the sequence's context_lens[b] positions, whose K/V must already be
 * in the pools (kv_cache_append with one slot per chunk token).  Row i of the
 * chunk, at position p = context_lens[b] - n_b + i, gets
 *
 *   out[row, h, :] = softmax_t(scale * q[row, h] . K_t) V_t  over t = 0..p,
 *
 * which is what unchunked causal attention over the whole prompt gives that
 * position.  A row with p < 0 (a chunk longer than its context) gets zeros.
 * A one-row chunk is a decode step.
 *
 *   out            [total_q, num_q_heads, head_dim] fp16 (16-byte aligned).
 *   q              [total_q, num_q_heads, head_dim] fp16, total_q =
 *                  query_start[B].
 *   query_start    [B + 1] int32, non-decreasing, query_start[0] = 0.
 *   max_query_len  >= every n_b (sizes the grid; rows of a longer chunk past
 *                  this bound are not written).  0 makes the call a no-op.
 * Other arguments, ranges and device-data guards as for
 * paged_attention_decode.
 */
int paged_attention_prefill(void* out, const void* q,
                            const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* query_start, int32_t B, int32_t max_query_len,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, float scale, void* stream);

/*
 * paged_attention_prefill_split -- paged_attention_prefill with each
 * sequence's context cut into partitions of partition_size positions (the
 * split of paged_attention_decode_split applied to a chunk's rows), for short
 * chunks over long contexts, where one workgroup per query tile streams the
 * whole context alone.  Merge with split_reduce over the chunk rows:
 * split_reduce(out, lse_out, partial_out, partial_lse, row_context_lens,
 * total_q, num_q_heads, head_dim, partition_size, max_partitions).
 *
 *   partial_out       [total_q, num_q_heads, max_partitions, head_dim] fp32
 *   partial_lse       [total_q, num_q_heads, max_partitions] fp32 workspace,
 *                     as paged_attention_decode_split's per chunk row: for a
 *                     row that sees no position of a partition that exists
 *                     for its sequence, lse = -inf and a zero row.
 *   row_context_lens  [total_q] int32 out: row r of sequence b gets
 *                     context_lens[b] (clamped), the length split_reduce needs
 *                     to count the row's partitions.  Rows past
 *                     query_start[B] are not written.
 * Other arguments as paged_attention_prefill, plus partition_size (a multiple
 * of block_size) and max_partitions (max_partitions * partition_size >=
 * max_blocks_per_seq * block_size).  The merged result equals
 * paged_attention_prefill up to fp32 summation order.
 */
int paged_attention_prefill_split(float* partial_out, float* partial_lse,
                                  int32_t* row_context_lens, const void* q,
                                  const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, int32_t B,
                                  int32_t max_query_len, int32_t num_q_heads,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t num_blocks, int32_t max_blocks_per_seq,
                                  int32_t partition_size, int32_t max_partitions, float scale,
                                  void* stream);

/*
 * split_reduce -- merge the partitions written by
 * paged_attention_decode_split.  With n = ceil(context_lens[b] /
 * partition_size) valid partitions of (b, h):
 *
 *   L          = ln(sum_{p<n} exp(partial_lse[b, h, p]))
 *   out[b,h,:] = sum_{p<n} exp(partial_lse[b, h, p] - L) partial_out[b,h,p,:]
 *
 * which equals the unsplit softmax result exactly in real arithmetic (the
 * pages name the split arm but not its merge; this log-sum-exp weighting is
 * the exact one).  context_lens[b] == 0 gives zeros and L = -inf.
 *
 *   out       [B, num_q_heads, head_dim] fp16 (written).
 *   lse_out   [B, num_q_heads] fp32 natural-log LSE of the whole context, or
 *             NULL.
 * Other arguments as for paged_attention_decode_split.
 */
int split_reduce(void* out, float* lse_out,
                 const float* partial_out, const float* partial_lse,
                 const int32_t* context_lens,
                 int32_t B, int32_t num_q_heads, int32_t head_dim,
                 int32_t partition_size, int32_t max_partitions, void* stream);

/* ------------------------------------------------------------------------
 * 8-bit KV cache.
 *
 * The pages mention an 8-bit KV cache only for another system (llama.cpp's
 * q8 cache for Gemma on an RTX 4090, Inference Engineering thread) and give
 * no format; this library's is:
 *   k_codes, v_codes    [num_blocks, num_kv_heads, block_size, head_dim] int8
 *   k_scales, v_scales  [num_blocks, num_kv_heads, block_size] fp32
 * Both are head-major within a block (unlike the fp16 pools): the row of
 * position t of KV head h is codes[block_tables[b, t / block_size], h,
 * t % block_size, :], so one head's rows of a block are contiguous and a
 * pass that reads one head fetches no other head's bytes.
 * Each (token, KV head) row of head_dim values is quantised when written:
 * amax = max |x| (fp16 values in fp32), inv = 127 / amax and code =
 * rint(x * inv) (IEEE fp32 division and multiply, nearest-even; within
 * [-127, 127]), scale = amax / 127; a zero row has codes 0 and scale 0.  The
 * row's value is code * scale.  Attention over the 8-bit cache computes the
 * same softmax as paged_attention_decode over those values.  Arrays 16-byte
 * aligned.  The bytes per (token, head) row are head_dim + 4 instead of
 * 2 * head_dim.  new K/V rows must be finite.
 * ------------------------------------------------------------------------ */

/* Quantise and write new tokens' K/V rows (bit-exact with the rule above).
 * Arguments as kv_cache_append with the pools replaced by codes + scales. */
int kv_cache_append_q8(void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                       const void* k_new, const void* v_new, const int64_t* slot_mapping,
                       int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, void* stream);

/* paged_attention_decode over the 8-bit cache. */
int paged_attention_decode_q8(void* out, const void* q,
                              const void* k_codes, const void* v_codes,
                              const float* k_scales, const float* v_scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, float scale, void* stream);

/* paged_attention_decode_split over the 8-bit cache (merge with
 * split_reduce). */
int paged_attention_decode_split_q8(float* partial_out, float* partial_lse, const void* q,
                                    const void* k_codes, const void* v_codes,
                                    const float* k_scales, const float* v_scales,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                    int32_t max_blocks_per_seq, int32_t partition_size,
                                    int32_t max_partitions, float scale, void* stream);

/* paged_decode_step over the 8-bit cache: the quantising cache write of
 * kv_cache_append_q8, the split pass of paged_attention_decode_split_q8 and
 * the merge of split_reduce in one launch (the single-launch step of
 * paged_decode_step, for the 8-bit format above).
 *   k_codes, v_codes, k_scales, v_scales   the 8-bit cache, updated in place
 *                     by the append.
 *   k_new, v_new      [B, num_kv_heads, head_dim] fp16, finite: one new token
 *                     per sequence, quantised by the format's rule (codes and
 *                     scale bit-identical to kv_cache_append_q8's).
 * Every other argument, the workspace and its state between calls, the slot
 * rule (the slot of position context_lens[b] - 1, else undefined attention
 * over the new value) and the merge are as for paged_decode_step.  Results
 * equal kv_cache_append_q8 + paged_attention_decode_split_q8 + split_reduce up
 * to fp32 summation order. */
int paged_decode_step_q8(void* out, float* lse_out,
                         void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                         const void* q, const void* k_new, const void* v_new,
                         const int64_t* slot_mapping,
                         const int32_t* block_tables, const int32_t* context_lens,
                         float* partial_out, float* partial_lse, int32_t* counters,
                         int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t partition_size,
                         int32_t max_partitions, float scale, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator (host memory only; no GPU call).
 *
 * The cache's num_blocks blocks are handed out on demand from a FIFO queue of
 * free block ids kept on the host (Inference Engineering, Day 11 post on
 * vLLM: the KV cache manager takes a free block from its free-block queue
 * when a request needs more space).  Each sequence id in [0, max_seqs) owns a
 * block table of at most max_blocks_per_seq blocks and holds exactly
 * ceil(len / block_size) blocks for its len tokens, so the memory it wastes
 * is less than one block (nanoserve write-up, "What I built": the paged
 * cache's waste is bounded by one block per sequence).  The queue starts as
 * 0, 1, ..., num_blocks - 1; a freed sequence's blocks go to its back in
 * table order.  Token position t of a sequence has slot
 * table[t / block_size] * block_size + t % block_size, the slot_mapping value
 * kv_cache_append takes.
 *
 * Ownership: pkv_allocator_create allocates the handle (its only allocation)
 * and pkv_allocator_destroy frees it.  All output arrays are caller-owned
 * host memory.  A handle is not thread-safe; separate handles are
 * independent.  Calls that fail return a negative status and change nothing.
 * ------------------------------------------------------------------------ */
typedef struct pkv_block_allocator pkv_block_allocator;

/* New allocator, or NULL for a non-positive argument or out of memory. */
pkv_block_allocator* pkv_allocator_create(int32_t num_blocks, int32_t block_size,
                                          int32_t max_seqs, int32_t max_blocks_per_seq);
void pkv_allocator_destroy(pkv_block_allocator* a);

/* Blocks in the free queue (or PKV_ERR_INVALID_ARG for a NULL handle). */
int32_t pkv_allocator_num_free(const pkv_block_allocator* a);

/* Tokens sequence `seq` holds (or PKV_ERR_INVALID_ARG). */
int32_t pkv_allocator_context_len(const pkv_block_allocator* a, int32_t seq);

/* Grow `seq` by num_tokens positions, taking blocks from the queue as needed;
 * writes the new positions' slots to slot_mapping[0 .. num_tokens).
 * PKV_ERR_NO_SPACE if the queue or the sequence's table cannot hold them. */
int pkv_allocator_append_slots(pkv_block_allocator* a, int32_t seq, int32_t num_tokens,
                               int64_t* slot_mapping);

/* Return every block of `seq` to the queue; its length becomes 0. */
int pkv_allocator_free_seq(pkv_block_allocator* a, int32_t seq);

/* Copy `seq`'s block table into row[0 .. width), padded with -1;
 * PKV_ERR_INVALID_ARG if width is below the blocks it holds. */
int pkv_allocator_block_table(const pkv_block_allocator* a, int32_t seq, int32_t* row,
                              int32_t width);

/* One decode step for B distinct sequences: each grows by one token (its
 * slot in slot_mapping[b]); block_tables [B, width] and context_lens [B]
 * receive the tables and lengths after the growth, ready for
 * kv_cache_append + paged_attention_decode / paged_decode_step.  All or
 * nothing: PKV_ERR_NO_SPACE if the batch does not fit, PKV_ERR_INVALID_ARG
 * for a repeated or out-of-range id or a width below a table's blocks. */
int pkv_allocator_build_decode_batch(pkv_block_allocator* a, const int32_t* seqs, int32_t B,
                                     int32_t width, int64_t* slot_mapping,
                                     int32_t* block_tables, int32_t* context_lens);

/* One chunked-prefill pass: sequence seqs[b] grows by chunk_lens[b] tokens.
 * query_start [B + 1] receives the chunks' row offsets, slot_mapping
 * [query_start[B]] the chunk tokens' slots in row order, block_tables
 * [B, width] and context_lens [B] the state after the growth: the inputs of
 * kv_cache_append + paged_attention_prefill.  All or nothing, as above. */
int pkv_allocator_build_prefill_batch(pkv_block_allocator* a, const int32_t* seqs,
                                      const int32_t* chunk_lens, int32_t B, int32_t width,
                                      int32_t* query_start, int64_t* slot_mapping,
                                      int32_t* block_tables, int32_t* context_lens);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
