/*
 * pa.h — C ABI of libpa.so: decode-step paged attention on a block-paged KV cache, for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [Visualized] "PagedAttention, Visualized" (penny-xu.github.io), Parts 2-3.
 *   [Digest]     "PagedAttention" (devoured.fyi digest), sections "PagedAttention in one picture",
 *                "Copy-on-write: when two requests share a prefix", "Why the attention kernel works
 *                at all", "Misconceptions".
 *   [Lesson06]   "LLM Inference Visualizer, Lesson 06: PagedAttention" (vivekgupta.ai), live
 *                diagram "How paging grows".
 *
 * What the library computes.  The KV cache of every running sequence lives in a shared pool of
 * fixed-size physical blocks of 16 token positions ([Digest] "PagedAttention in one picture";
 * [Visualized] Part 3 table, "Block (16 tokens)").  A per-sequence block table maps logical block
 * j (token positions 16j .. 16j+15) to a physical block id ([Digest] same section: an entry 7 at
 * index 0 puts the first 16 positions of that sequence in physical block 7).  Decode attention walks that table and
 * gathers K and V from wherever the blocks landed; the result is exactly ordinary attention on the
 * de-paged sequence ([Digest] "Misconceptions": the math is untouched).
 *
 * Conventions for every entry point below.
 *  - All device memory is owned by the caller.  The library never allocates, frees or
 *    synchronises device memory; it only enqueues kernels on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream).  Every call returns before the work has run.
 *  - Host-side validation runs before any launch; on failure nothing is enqueued and the call
 *    returns a negative pa_status; pa_last_error() then holds a thread-local description.
 *  - After a launch, a HIP launch error is returned as PA_ERR_LAUNCH.
 *  - Functions are re-entrant.  Global state: the thread-local error text, the process-wide
 *    PA_DEBUG switch, per-device values looked up once (compute units, the kernels' occupancy,
 *    the address of pa_decode_attention_noalloc's scratch) and that scratch itself.
 *  - Calls that touch the same device buffers on different streams race; order them yourself.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                                        */
  PA_ERR_SHAPE = -2,       /* sizes are negative or inconsistent with each other                */
  PA_ERR_UNSUPPORTED = -3, /* a valid request this build does not implement (dtype, head_dim...) */
  PA_ERR_WORKSPACE = -4,   /* the workspace is smaller than pa_decode_workspace_bytes()         */
  PA_ERR_ALIAS = -5,       /* copy pairs overlap (a destination repeats or is also a source)    */
  PA_ERR_LAUNCH = -6,      /* HIP reported an error when the kernels were enqueued              */
  PA_ERR_NO_BLOCKS = -7,   /* block manager: the free list is empty                             */
  PA_ERR_STATE = -8        /* block manager: unknown sequence or block id                       */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,      /* IEEE binary32                                                          */
  PA_F16 = 1,      /* IEEE binary16                                                          */
  PA_BF16 = 2,     /* bfloat16 (upper half of binary32)                                      */
  PA_FP8_E4M3 = 3  /* OCP FP8 E4M3FN: bias 7, no infinities, NaN = S.1111.111, max +-448;
                      cache storage only, always with one fp32 scale per KV head             */
} pa_dtype;

/* The default block size: 16 token positions per block, the default the pages give ([Digest]
 * "PagedAttention in one picture" and "Misconceptions").  Pools of 8 or 32 positions per block are
 * accepted where a function says so: the pages describe the block size as a tradeoff between the
 * padding in each sequence's last block and the table size and per-block overhead ([Digest]
 * "Misconceptions"). */
#define PA_BLOCK_SIZE 16

/*
 * One layer's KV cache.  k_pool and v_pool are device buffers of pa_pool_bytes() bytes each.
 *
 * Pool layout (owned by the library; described here so that independent code can read it).
 * Let e be the element size of cache_dtype in bytes (f32 4, f16 2, bf16 2, fp8 1), E = 16 / e the
 * number of elements in one 16-byte vector, B = block_size (8, 16 or 32), D = head_dim,
 * H = num_kv_heads.
 * Both pools are block-major and then head-major: block b holds H consecutive tiles, one per KV
 * head, each of B*D elements (B*D*e bytes: 4 KiB for f16/bf16 at D = 128, always a whole number
 * of 128-byte lines).  Tile (b, h) starts at element (b*H + h) * B*D.  Inside a tile:
 *
 *   K tile: the head dimension is cut into D/E vectors of E elements (16 bytes).  Vector c of token
 *           slot t is stored at vector index c*B + t, so element (t, i) sits at element offset
 *           ((i / E) * B + t) * E + (i % E) within the tile.  One 16-byte vector per token, for all
 *           B tokens, forms 16 * B contiguous bytes.
 *   V tile: stored transposed: the B values of head-dimension index i are contiguous, so element
 *           (t, i) sits at element offset i * B + t within the tile.
 *
 * Token position p of a sequence with block table `bt` lives in block bt[p / B] at slot t = p % B;
 * its global slot number is bt[p / B] * B + p % B (the slot_mapping value used by
 * pa_reshape_and_cache).
 *
 * fp8: an element stored as byte c represents decode(c) * scale[h], where decode is the E4M3FN value
 * of c and scale = k_scale for the K pool, v_scale for the V pool (device arrays of num_kv_heads
 * fp32 values, one per KV head of this layer).  For the other dtypes the scale pointers must be NULL.
 */
typedef struct pa_cache {
  void *k_pool;            /* device, pa_pool_bytes() bytes                       */
  void *v_pool;            /* device, pa_pool_bytes() bytes                       */
  const float *k_scale;    /* device [num_kv_heads] fp32, fp8 only, else NULL      */
  const float *v_scale;    /* device [num_kv_heads] fp32, fp8 only, else NULL      */
  int32_t num_blocks;      /* physical blocks in this pool                        */
  int32_t block_size;      /* 8, 16 (PA_BLOCK_SIZE) or 32, see each function       */
  int32_t num_kv_heads;    /* 1 .. 16                                             */
  int32_t head_dim;        /* 64 or 128                                           */
  int32_t cache_dtype;     /* a pa_dtype                                          */
} pa_cache;

/* Bytes of ONE of k_pool / v_pool: num_blocks * num_kv_heads * block_size * head_dim * e.
 * Returns 0 for an invalid description.  For Qwen2.5-7B-shaped layers (4 KV heads, head_dim 128,
 * f16) 2 * pa_pool_bytes / (num_blocks * 16) is 2,048 bytes per token per layer, i.e. 57,344 bytes
 * per token over 28 layers ([Visualized] Part 2). */
size_t pa_pool_bytes(const pa_cache *cache);

/*
 * pa_reshape_and_cache — write each new token's K and V into its slot.
 * A new token's K and V go to the next unused slot of its sequence's last block ([Lesson06] "How
 * paging grows"), where every later token reads them ([Visualized] Part 2).
 *
 *   key, value    device [num_tokens] rows; row t holds num_kv_heads * head_dim elements of
 *                 `in_dtype` laid out [kv_head][head_dim]; consecutive rows are key_stride /
 *                 value_stride ELEMENTS apart (>= num_kv_heads * head_dim).
 *   slot_mapping  device int64 [num_tokens]: token t goes to block slot_mapping[t] / B, slot
 *                 slot_mapping[t] % B (B = block_size: 8, 16 or 32).  A negative value skips the
 *                 token (padding); a value >= num_blocks * B is also skipped and never written.
 *   in_dtype      f32/f16/bf16.  For an f32/f16/bf16 cache it must equal cache_dtype and the
 *                 element is copied bit for bit.  For an fp8 cache each element x becomes
 *                 E4M3FN(round-to-nearest-even, saturating at +-448)(float(x) / scale[h]), the
 *                 division done in IEEE fp32; NaN becomes 0x7F with the sign of x.
 * Two tokens with the same slot in one call race; callers must not do that.
 */
pa_status pa_reshape_and_cache(const pa_cache *cache, const void *key, const void *value,
                               int32_t in_dtype, int64_t key_stride, int64_t value_stride,
                               const int64_t *slot_mapping, int32_t num_tokens, void *stream);

/* Partition size used when pa_decode_attention is given partition_size = 0 for these sizes:
 * 1,024 positions for at most 64 (sequence, KV head) rows with contexts of 4,096 or more; 512 for
 * 2,048 rows or more with contexts of 8,192 or more; else 256 halved (down to 64) while that
 * leaves fewer than 512 partitions in all. */
int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len);

/* Device workspace bytes pa_decode_attention needs for these sizes (0 is a valid answer when the
 * work fits one partition per sequence).  partition_size = 0 means the automatic choice. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/* Flags for pa_decode_attention. */
#define PA_DECODE_DEFAULT 0u
#define PA_DECODE_FORCE_VALU 1u  /* use the vector-ALU kernel even where the matrix-core one applies */
#define PA_DECODE_PLAN_APPEND 2u /* pa_decode_plan only: plan for pa_decode_attention_append's grid */

/*
 * pa_decode_attention — one decode step of paged attention for a batch of sequences.
 * The kernel walks each sequence's block table and gathers K and V block by block ([Digest]
 * "PagedAttention in one picture", "Why the attention kernel works at all"); the result is the
 * ordinary attention of the de-paged sequence ([Digest] "Misconceptions"):
 *
 *   for sequence s with L = context_lens[s] and query head q (KV head h = q / (num_q_heads /
 *   num_kv_heads)):  z_p = scale * <query[s][q], K_s[p][h]> for p in [0, L);
 *   out[s][q] = sum_p exp(z_p - max z) * V_s[p][h] / sum_p exp(z_p - max z);   out = 0 when L == 0,
 *   where K_s[p][h] is element (slot p % B) of tile (block_tables[s][p / B], h) of the K pool,
 *   B = block_size.
 *
 *   out           device [num_seqs][num_q_heads][head_dim] in q_dtype, written in full.
 *   query         device rows of num_q_heads * head_dim elements of q_dtype; sequence s starts at
 *                 element s * q_stride (q_stride 0 means num_q_heads * head_dim).
 *   q_dtype       f32 with an f32 cache; f16 with an f16 cache; bf16 with a bf16 cache; f16 or
 *                 bf16 with an fp8 cache.
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq].  Only the first ceil(L / B)
 *                 entries of row s are read; the rest may hold anything.  An entry outside
 *                 [0, num_blocks) is never dereferenced: the B positions it covers are left out.
 *   context_lens  device int32 [num_seqs]; L includes the token written this step.  Values are
 *                 clamped to [0, min(max_context_len, B * max_blocks_per_seq)].
 *   seq_order     NULL, or device int32 [num_seqs] holding each of 0 .. num_seqs - 1 once: the
 *                 order in which the sequences' work is dealt to the device's wavefronts
 *                 (pa_decode_plan computes a balanced one from the host's copy of the context
 *                 lengths).  It changes the time of the call, never its result: the output is the
 *                 same bit for bit with any permutation.  An entry outside 0 .. num_seqs - 1 is
 *                 skipped, and a sequence that no entry names gets undefined output (PA_DEBUG
 *                 checks that the array is a permutation).  Used by the matrix-core kernel's
 *                 persistent grid (at most 4,096 sequences; 2,048 with a shared prefix) while
 *                 num_seqs times the partitions of the longest row stays below 2^20; ignored
 *                 elsewhere.
 *   max_context_len  host upper bound of context_lens, used to size the launch without reading
 *                 the device.
 *   scale         softmax scale, normally 1 / sqrt(head_dim).
 *   partition_size  most tokens per split-K partition: 0 = pa_decode_auto_partition(),
 *                 otherwise a positive multiple of 16.  A context of L tokens is cut into
 *                 ceil(L / partition_size) partitions of whole 16-position steps, as equal as
 *                 those allow (a partition may start inside a 32-position block); when there are
 *                 several they are computed independently (each keeps its running max, running
 *                 sum and output, and stores the max, the sum and its normalised output) and
 *                 merged by a second kernel.  Where the call's rows hold between one and two
 *                 partitions per SIMD of the device, one wavefront computes two consecutive
 *                 partitions of a row in one pass over their blocks; each still stores its own
 *                 partial.  pa_decode_plan can pick a larger size for automatic calls.
 *   workspace     device scratch of at least pa_decode_workspace_bytes() bytes (NULL if 0).
 * Arithmetic: products, exponentials and sums in fp32 (the matrix cores take f16 / bf16 operands,
 * fp8 codes widened to f16); the result rounds once to q_dtype.  With f16 queries on the matrix
 * cores each partition's normalised output is kept in fp16 (round to nearest even) until the
 * merge, adding at most 2^-11 of its magnitude; with an fp8 cache it is kept in units of the codes
 * (|x| <= 448) and the head's v_scale is applied after the merge, so no partial overflows.
 * Supported: head_dim 64 or 128, num_q_heads a multiple of num_kv_heads with at most 16 query
 * heads per KV head; block_size 16 for every dtype, 8 or 32 for the matrix-core configurations
 * (f16 / bf16 caches with the same query dtype, fp8 caches with f16 queries, 16-byte aligned query
 * rows, 8-byte aligned output), 8 only for pools below 4 GiB.  Anything else is
 * PA_ERR_UNSUPPORTED.
 */
pa_status pa_decode_attention(void *out, const void *query, int32_t q_dtype, int64_t q_stride,
                              const pa_cache *cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              const int32_t *seq_order, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              void *workspace, size_t workspace_bytes, uint32_t flags,
                              void *stream);

/*
 * pa_decode_plan — a dealing order for pa_decode_attention's seq_order, computed on the host
 * from a HOST copy of the step's context lengths: step metadata that the scheduler holds beside
 * the block tables the kernel walks ([Digest] "PagedAttention in one picture"), while the order
 * only changes how the kernel fetches, not the attention it computes ([Digest] "Misconceptions").
 * Every sequence's positions are cut into partitions (work items) as the call cuts them; the
 * sequences are taken by the size of their largest item, largest first, and put into rounds of as
 * many items as the call's grid has wavefronts for them, the rounds filled alternately from the
 * largest and from the smallest sequences left, so that a wavefront dealt a large item in one round
 * gets a small one in the next and the wavefronts end close together (with at most two rounds:
 * the largest sequences on the wavefronts that take one item, the next largest in the first round
 * of the others, the rest smallest first).  The call's partition reduce merges rows in the same
 * order.
 *   cache, q_dtype, num_q_heads, max_blocks_per_seq, max_context_len, prefix_len,
 *   partition_size  those of the decode call the order is for (prefix_len 0: pa_decode_attention;
 *                 > 0: pa_decode_attention_shared_prefix).
 *   context_lens  HOST int32 [num_seqs], clamped as the call clamps them.
 *   flags         PA_DECODE_FORCE_VALU as in the call; PA_DECODE_PLAN_APPEND for the grid of
 *                 pa_decode_attention_append.
 *   seq_order     HOST int32 [num_seqs], written: a permutation of 0 .. num_seqs - 1 (the identity
 *                 where the call would not deal a list or ignores the order: the vector-ALU
 *                 kernel, the direct grid, 2^20 or more partition slots in all; and where no
 *                 order balances anything: the items fill at most half of one round, or, without
 *                 a shared prefix, at most one round).
 *   round_items   optional (NULL): the items per round, the grid's wavefronts that take sequence
 *                 items on the current device (0 with the identity).
 *   partition_size_out  optional (NULL): the partition_size to make the call with, for which the
 *                 order was planned.  The caller's own partition_size, except where it is 0
 *                 (automatic) for a call without a shared prefix whose list takes more than one
 *                 round: then the planner also tries larger partitions (multiples of 64 positions
 *                 above the automatic size, up to 2,048, while the list keeps more than one round)
 *                 and returns the one whose planned deal has the least busiest-wavefront KV bytes
 *                 plus 240 KiB per round of items (fewer items: fewer ring fills, partials and
 *                 merges; a measured trade-off), or 0 where the automatic size wins.  A size the
 *                 planner returns is never below the automatic one, so a workspace sized for
 *                 partition_size 0 still suffices.
 * The grid depends on the current device (its compute units); an order planned for another
 * device, or for other lengths, is still a valid seq_order, only less balanced.
 */
pa_status pa_decode_plan(const pa_cache *cache, int32_t q_dtype, const int32_t *context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int32_t prefix_len, int32_t partition_size,
                         uint32_t flags, int32_t *seq_order, int32_t *round_items,
                         int32_t *partition_size_out);

/*
 * pa_decode_attention_noalloc — pa_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The split-K partials go to a fixed scratch array of
 * PA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU it runs on until the
 * process ends; the call itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine) and its first call on a device looks up that device's copy of the array.
 *   All arguments and results are those of pa_decode_attention with seq_order NULL (same
 *   kernels, same partition sizes, bit-identical output).
 *   A call whose partials need more than PA_NOALLOC_SCRATCH_BYTES (the need is at most
 *   pa_decode_workspace_bytes() for the same sizes) returns PA_ERR_WORKSPACE before touching the
 *   device; so do all the argument errors of pa_decode_attention.
 *   Every call on one GPU shares that GPU's scratch, and nothing in it needs to start at zero
 *   (each call reads only the partials it wrote): calls that overlap on one GPU (different streams
 *   or threads without ordering) race; order them yourself.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
pa_status pa_decode_attention_noalloc(void *out, const void *query, int32_t q_dtype,
                                      int64_t q_stride, const pa_cache *cache,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len, float scale,
                                      int32_t partition_size, uint32_t flags, void *stream);

/*
 * pa_decode_attention_shared_prefix — pa_decode_attention for a batch whose sequences all begin
 * with the same prefix_len positions stored in the same physical blocks: several requests share a
 * prompt prefix and their block tables point at one copy of it ([Visualized] Part 3, shared
 * prefix blocks with a reference count; [Digest] "Copy-on-write: when two requests share a
 * prefix" and "Misconceptions", on system prompts shared by many users).  The result is the same
 * attention as pa_decode_attention over each sequence's whole context (within floating-point
 * rounding: the summation order differs); only the reading changes: each block of the prefix is
 * read for groups of 64 (sequence, query head) rows at a time, staged once per group in on-chip
 * memory, instead of once per sequence.
 *
 *   prefix_table  device int32 [prefix_len / 16]: the prefix's physical block ids.  The first
 *                 prefix_len / 16 entries of every block_tables row must hold the same ids (the
 *                 caller's guarantee; they are what the sharing means).
 *   prefix_len    shared positions, a non-negative multiple of 16 (0: plain decode).  A sequence
 *                 whose context length is below prefix_len attends only to its first
 *                 context_lens[s] positions, as in pa_decode_attention.
 *   workspace     at least pa_decode_shared_prefix_workspace_bytes() bytes.
 * The prefix is computed in chunks of 512 positions; the positions after it are cut into
 * partitions as in pa_decode_attention (ceil((L - prefix_len) / partition_size) of them).
 * All other arguments and rules are those of pa_decode_attention.  The prefix path runs on
 * 16-position blocks; batches it does not cover (8- or 32-position blocks, more than 2048
 * sequences, the vector-ALU dtype pairs, PA_DECODE_FORCE_VALU) are computed by the plain decode,
 * with the same result: each sequence then reads the prefix through its own table, and
 * prefix_table is checked but not read.
 */
pa_status pa_decode_attention_shared_prefix(void *out, const void *query, int32_t q_dtype,
                                            int64_t q_stride, const pa_cache *cache,
                                            const int32_t *block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t *context_lens,
                                            const int32_t *seq_order, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t max_context_len,
                                            float scale, const int32_t *prefix_table,
                                            int32_t prefix_len, int32_t partition_size,
                                            void *workspace, size_t workspace_bytes,
                                            uint32_t flags, void *stream);

/*
 * pa_decode_attention_append — one decode step with its cache write: pa_reshape_and_cache of each
 * sequence's new token followed by pa_decode_attention (prefix_len = 0) or
 * pa_decode_attention_shared_prefix (prefix_len > 0), in one call.  The step's new K and V land
 * in the next free slot of the sequence's last block ([Lesson06] "How paging grows"), and the
 * same step's query already attends to them, as position context_lens[s] - 1 ([Visualized]
 * Parts 1 and 2).
 *
 *   key, value    device rows of num_kv_heads * head_dim elements of q_dtype, one per sequence;
 *                 sequence s's row starts at element s * key_stride (value_stride); a stride of
 *                 0 means num_kv_heads * head_dim.  Written into the cache as
 *                 pa_reshape_and_cache writes rows of that dtype (a bit copy, or E4M3FN with the
 *                 per-head scales for an fp8 cache).
 *   slot_mapping  device int64 [num_seqs]: the slot of position context_lens[s] - 1 of sequence s
 *                 (its block table's entry for that position times block_size, plus the offset),
 *                 or negative for no write.  With a shared prefix the position must lie after it
 *                 (context_lens[s] > prefix_len); a slot given for a shorter context is not
 *                 written (and its attention reads position context_lens[s] - 1 from the pool).
 *                 Two sequences must not share a slot.  With prefix_len > 0 the call needs the
 *                 matrix-core kernel (the prefix path, or the plain decode for the batches the
 *                 prefix path does not cover): the vector-ALU configurations are
 *                 PA_ERR_UNSUPPORTED, and nothing is written.
 *   prefix_table, prefix_len  as in pa_decode_attention_shared_prefix (NULL / 0: plain decode).
 *   workspace     at least pa_decode_workspace_bytes() (pa_decode_shared_prefix_workspace_bytes()
 *                 with a prefix) bytes.
 * All other arguments and rules are those of pa_decode_attention.  The pools end byte for byte as
 * pa_reshape_and_cache leaves them.  On the matrix-core kernel the wavefront that walks the last
 * positions of each (sequence, KV head) writes that head's part of the token and takes the token
 * from registers instead of reading it back, so one kernel does both; the attention equals that of
 * the two calls within floating-point rounding (the new position is summed last).  Configurations
 * of the vector-ALU kernel, and key/value rows that are not 4-byte aligned, run the two calls;
 * with a shared prefix, rows that are not 4-byte aligned (or odd strides) are PA_ERR_SHAPE.
 */
pa_status pa_decode_attention_append(void *out, const void *query, int32_t q_dtype,
                                     int64_t q_stride, const pa_cache *cache, const void *key,
                                     const void *value, int64_t key_stride, int64_t value_stride,
                                     const int64_t *slot_mapping, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, const int32_t *context_lens,
                                     const int32_t *seq_order, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_context_len, float scale,
                                     const int32_t *prefix_table, int32_t prefix_len,
                                     int32_t partition_size, void *workspace,
                                     size_t workspace_bytes, uint32_t flags, void *stream);

/* Device workspace bytes pa_decode_attention_shared_prefix needs for these sizes. */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t prefix_len,
                                               int32_t partition_size);

/*
 * pa_prefill_attention — paged attention for a chunk of new tokens per sequence: a prompt, or a
 * piece of one.  A prompt goes through the model as one matrix whose tokens look at each other,
 * and a token's K and V serve every token after it ([Visualized] Parts 1 and 2): sequence s has
 * n_s = query_start[s+1] - query_start[s] new tokens at positions L_s - n_s .. L_s - 1
 * (L_s = context_lens[s], the new tokens already written by pa_reshape_and_cache), and the token at
 * position p attends to positions 0 .. p of its sequence, through its block table.
 *
 *   out           device [num_tokens][num_q_heads][head_dim], query dtype, written for every new
 *                 token of every sequence.
 *   query         device [num_tokens][num_q_heads][head_dim]; token rows q_stride elements apart
 *                 (0 = packed).
 *   query_start   device int32 [num_seqs + 1]: query_start[0] = 0, non-decreasing, the last one
 *                 num_tokens; n_s <= L_s.
 *   max_query_len host upper bound of every n_s (sizes the grid; larger n_s are cut to it).
 *   Other arguments as in pa_decode_attention.  No workspace: each token's rows are computed
 *   whole by one wavefront.
 * Supported: block_size 16 and the matrix-core configurations of pa_decode_attention (f16 / bf16
 * caches with the same query dtype, fp8 caches with f16 queries; head_dim 64 or 128; at most 16
 * query heads per KV head; 16-byte aligned query rows and q_stride a multiple of 8; 8-byte aligned
 * output); anything else is PA_ERR_UNSUPPORTED.
 */
pa_status pa_prefill_attention(void *out, const void *query, int32_t q_dtype, int64_t q_stride,
                               const pa_cache *cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               const int32_t *query_start, int32_t num_seqs, int32_t num_tokens,
                               int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                               float scale, void *stream);

/*
 * pa_copy_blocks — the clone step of copy-on-write.  When a sequence must write into a block
 * whose reference count is above 1, the engine clones that block, drops the original's count by
 * one and points the writer's table at the clone ([Digest] "Copy-on-write: when two requests share
 * a prefix"; [Visualized] Part 3, "Copy-on-write after fork()").  For every (src, dst) pair and
 * every layer this copies all KV heads of block src to block dst in both pools, bit for bit.
 *
 *   layers        HOST array of num_layers pa_cache descriptions with identical shape and dtype.
 *   block_pairs   device int32 [num_pairs][2] = {src, dst}.  Destinations must be distinct and no
 *                 destination may also be a source in the same call (a fresh clone target);
 *                 pairs with an id outside [0, num_blocks) are skipped.
 */
pa_status pa_copy_blocks(const pa_cache *layers, int32_t num_layers, const int32_t *block_pairs,
                         int32_t num_pairs, void *stream);

/* Host-side check of the copy-pair rules above on a HOST copy of block_pairs: PA_ERR_ALIAS when a
 * destination repeats or is also a source, PA_ERR_SHAPE when an id is out of range. */
pa_status pa_check_copy_pairs(const int32_t *block_pairs_host, int32_t num_pairs,
                              int32_t num_blocks);

/* Host-side check of a HOST copy of a slot_mapping: PA_ERR_ALIAS when two tokens name the same
 * slot (a race in pa_reshape_and_cache); slots that are negative or past the pool are skipped, as
 * the kernels skip them. */
pa_status pa_check_slots(const int64_t *slots_host, int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size);

/* Host-side check of a HOST copy of context_lens: PA_ERR_SHAPE when a length is negative or above
 * max_context_len (the host bound that sizes the decode's launch). */
pa_status pa_check_context_lens(const int32_t *context_lens_host, int32_t num_seqs,
                                int32_t max_context_len);

/* Host-side check of a HOST copy of a seq_order: PA_ERR_SHAPE unless it holds each of
 * 0 .. num_seqs - 1 exactly once. */
pa_status pa_check_seq_order(const int32_t *seq_order_host, int32_t num_seqs);

/*
 * Debug checks (PA_DEBUG).  Off by default; on when the environment variable PA_DEBUG is set to a
 * non-zero value at the library's first use, or after pa_set_debug(1).  With them on, before
 * anything is enqueued:
 *   pa_reshape_and_cache and pa_decode_attention_append copy slot_mapping to the host and run
 *     pa_check_slots (repeated slots: PA_ERR_ALIAS);
 *   pa_copy_blocks copies block_pairs to the host and runs pa_check_copy_pairs (PA_ERR_ALIAS,
 *     PA_ERR_SHAPE);
 *   every decode entry point copies context_lens to the host and runs pa_check_context_lens
 *     (PA_ERR_SHAPE), and a seq_order, when given, with pa_check_seq_order (PA_ERR_SHAPE).
 * The copies wait for the stream to reach the call (hipStreamSynchronize), so debug mode gives up
 * the library's rule of never synchronising; a failed check enqueues nothing.  The switch is
 * process-wide.
 */
void pa_set_debug(int on);
int pa_debug_enabled(void);

/*
 * pa_swap_blocks — evicting blocks to CPU memory and bringing them back, the KV cache's swapping
 * to disk ([Visualized] Part 3, the OS-to-PagedAttention table and the paragraph after it).  For
 * every (device block, host slot) pair and every layer, all KV heads of the device block are copied
 * to the host slot (to_host != 0) or the host slot's bytes back to the device block (to_host == 0),
 * in both pools, bit for bit.  The pairs come from pa_bm_swap_out / pa_bm_swap_in.
 *
 *   layers        HOST array of num_layers pa_cache descriptions with identical shape and dtype.
 *   host_k, host_v  HOST arrays of num_layers pointers to pinned host memory (hipHostMalloc /
 *                 torch pin_memory) of num_host_blocks * block bytes each, a block laid out as in
 *                 the device pool (block bytes = pa_pool_bytes / num_blocks).  The library checks
 *                 with hipPointerGetAttributes that the device can reach each one and refuses the
 *                 call otherwise (PA_ERR_UNSUPPORTED).
 *   block_pairs   int32 [num_pairs][2] = {device block, host slot} in device memory or pinned host
 *                 memory; pairs with an id outside [0, num_blocks) or [0, num_host_blocks) are
 *                 skipped.  Device blocks must be distinct, and host slots too (a race otherwise).
 * The copy is enqueued on `stream` like every other call; the host side of a swap-out may be read
 * only after the stream has reached it.
 */
pa_status pa_swap_blocks(const pa_cache *layers, int32_t num_layers, void *const *host_k,
                         void *const *host_v, int32_t num_host_blocks, const int32_t *block_pairs,
                         int32_t num_pairs, int32_t to_host, void *stream);

const char *pa_status_string(pa_status status);
const char *pa_last_error(void); /* thread-local text of the last failure on this thread */

/* ------------------------------------------------------------------------------------------
 * Host block manager (no GPU calls).  It owns the free list, per-block reference counts and the
 * per-sequence block tables, and produces the step metadata the kernels consume: slot numbers,
 * block tables, context lengths and copy-on-write pairs.
 *   - Blocks are handed out one at a time, only when a sequence's last block is full
 *     ([Lesson06] "How paging grows"; [Digest] table row "page fault / alloc").
 *   - A finished sequence's blocks go back to the pool ([Digest] "PagedAttention in one picture").
 *   - fork() makes a child whose table points at all of the parent's blocks, each reference count
 *     +1 ([Visualized] Part 3 shared prefix blocks; [Digest] copy-on-write section).
 *   - append() into a block whose count is above 1 clones it first ([Digest] copy-on-write).
 *   - swap_out() evicts a sequence's blocks to host slots, except the shared ones, which stay on
 *     the device because another sequence still needs them; swap_in() brings them back
 *     ([Visualized] Part 3, OS table: swapping to disk is evicting blocks to CPU memory).
 * Free lists: stacks.  The initial device order is given by the caller (free_order[0] is handed
 * out first), host slots are handed out 0, 1, 2, ... at first; a freed entry is pushed on top and
 * is the next one handed out.
 * ------------------------------------------------------------------------------------------ */
typedef struct pa_bm pa_bm;

/* free_order: HOST int32 [num_blocks], a permutation of 0..num_blocks-1 (NULL = 0, 1, 2, ...).
 * Returns NULL on invalid arguments or allocation failure. */
pa_bm *pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order);
void pa_bm_destroy(pa_bm *bm);

/* New empty sequence; ids are 0, 1, 2, ... in creation order and are never reused. */
pa_status pa_bm_add_seq(pa_bm *bm, int32_t *seq_id);

/* New sequence sharing every block of `parent` (each block's count +1), same context length. */
pa_status pa_bm_fork(pa_bm *bm, int32_t parent, int32_t *child);

/* Append one token position to `seq`.  If its length L is a multiple of block_size a fresh block
 * is taken from the free list.  Otherwise, if the last block's count is above 1, a fresh block is
 * taken, (*cow_src, *cow_dst) = (old, fresh) is reported, the old block's count drops by one and
 * the table points at the fresh block; else *cow_src = *cow_dst = -1.  *slot receives
 * table[L / block_size] * block_size + L % block_size, then L grows by one.  On
 * PA_ERR_NO_BLOCKS nothing changes. */
pa_status pa_bm_append(pa_bm *bm, int32_t seq, int64_t *slot, int32_t *cow_src, int32_t *cow_dst);

/* pa_bm_append for seqs[0..n) in order.  slots[i] is seqs[i]'s slot; the copy pairs are written
 * to cow_pairs as {src, dst} rows in order of occurrence, *num_pairs of them (cow_pairs must hold
 * n rows).  Stops at the first failure; the appends before it stay done. */
pa_status pa_bm_append_batch(pa_bm *bm, const int32_t *seqs, int32_t n, int64_t *slots,
                             int32_t *cow_pairs, int32_t *num_pairs);

/* Release a sequence: every block's count drops by one; blocks reaching 0 return to the pool. */
pa_status pa_bm_free_seq(pa_bm *bm, int32_t seq);

int32_t pa_bm_refcount(const pa_bm *bm, int32_t block); /* -1 for a bad id */
int32_t pa_bm_num_free(const pa_bm *bm);
int32_t pa_bm_seq_len(const pa_bm *bm, int32_t seq);    /* context length, -1 for a bad id */

/* Host slots for swapped-out blocks: num_host_blocks of them, 0 handed out first.  PA_ERR_STATE
 * while a sequence is swapped out. */
pa_status pa_bm_set_host_blocks(pa_bm *bm, int32_t num_host_blocks);

/* Evict `seq` (resident): each table entry whose block has count 1, in table order, gets a host
 * slot; the pair {block, slot} is written to pairs (cap rows), the device block is freed and the
 * entry becomes the slot.  Shared blocks stay on the device and keep seq's reference.  *num_pairs
 * = the number of moves.  Nothing changes on PA_ERR_SHAPE (cap too small) or PA_ERR_NO_BLOCKS
 * (too few free host slots).  A swapped-out sequence cannot append, fork or be exported until
 * pa_bm_swap_in; pa_bm_free_seq returns its host slots. */
pa_status pa_bm_swap_out(pa_bm *bm, int32_t seq, int32_t *pairs, int32_t cap, int32_t *num_pairs);

/* Bring `seq` back: each host-slot entry, in table order, gets a fresh device block; the pair
 * {block, slot} is written to pairs, the slot is freed and the entry becomes the block.  Nothing
 * changes on PA_ERR_SHAPE (cap too small) or PA_ERR_NO_BLOCKS (too few free device blocks). */
pa_status pa_bm_swap_in(pa_bm *bm, int32_t seq, int32_t *pairs, int32_t cap, int32_t *num_pairs);

int32_t pa_bm_num_free_host(const pa_bm *bm);
int32_t pa_bm_is_swapped(const pa_bm *bm, int32_t seq); /* 1 out, 0 resident, -1 bad id */

/* Copy seq's table into out[0..cap); *num_blocks = its length in blocks (may exceed cap; only
 * min(cap, length) entries are written).  For a swapped-out sequence, entries that were moved hold
 * host slot ids. */
pa_status pa_bm_block_table(const pa_bm *bm, int32_t seq, int32_t *out, int32_t cap,
                            int32_t *num_blocks);

/* Rows of the kernels' block_tables / context_lens for seqs[0..n): tables is HOST int32
 * [n][max_blocks_per_seq], entries past a sequence's length set to pad_value; PA_ERR_SHAPE if a
 * table is longer than max_blocks_per_seq. */
pa_status pa_bm_export(const pa_bm *bm, const int32_t *seqs, int32_t n, int32_t *tables,
                       int32_t max_blocks_per_seq, int32_t pad_value, int32_t *context_lens);

#ifdef __cplusplus
}
#endif
#endif /* PA_H */
