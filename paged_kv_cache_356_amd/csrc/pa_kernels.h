// pa_kernels.h — host-side launch interface between the C ABI layer (pa_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by pa_api.cpp and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

constexpr int kBlock = 16;  // token positions per KV block by default, and per ring step

// Shared-prefix decode: prefix positions per prefix work item (and per workspace partition slot);
// 256 and 1,024 measured slower on the 1,024-position prefix of 256 sequences.
constexpr int32_t kPrefixChunk = 512;

inline int dtype_bytes(int dt) {
  return dt == kF32 ? 4 : (dt == kF16 || dt == kBF16) ? 2 : dt == kFP8 ? 1 : 0;
}

struct CacheArgs {
  void *k_pool;
  void *v_pool;
  const float *k_scale;
  const float *v_scale;
  int32_t num_blocks;
  int32_t block_size;  // token positions per block: 8, 16 or 32 (16 unless stated otherwise)
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
};

struct ReshapeArgs {
  CacheArgs cache;
  const void *key;
  const void *value;
  int32_t in_dtype;
  int64_t key_stride;    // elements between token rows
  int64_t value_stride;  // elements between token rows
  const int64_t *slots;
  int32_t num_tokens;
};

// Per-partition results of the split-K decode, owned by the caller's workspace:
//   part_out [S][Hq][P][D] fp32, normalised partial outputs
//   part_ml  [S][Hq][P][2] fp32, (running max, running sum) of each partition
struct DecodeArgs {
  void *out;
  const void *q;
  int64_t q_stride;
  int32_t q_dtype;
  CacheArgs cache;
  const int32_t *block_tables;
  int32_t max_blocks_per_seq;
  const int32_t *context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_context_len;  // already clamped to 16 * max_blocks_per_seq
  float scale;
  int32_t partition_size;   // tokens per partition, multiple of 16
  int32_t num_partitions;   // ceil(max_context_len / partition_size)
  float *part_out;          // NULL when num_partitions == 1
  int32_t part_f16;         // 1: part_out holds fp16 values (matrix-core kernel, f16 queries)
  int32_t part_vscale;      // 1: those values are in fp8 code units; the reduce applies v_scale
  float *part_ml;
  int32_t persistent;       // grid mode of the matrix-core kernel (set by its launcher)
  int32_t num_cus;          // compute units of the device (set by the launcher; 0: unknown)
  // Paired items (set by the matrix-core launcher; plain decode only): a wavefront's item is two
  // consecutive partitions of one (sequence, KV head) row, streamed as one run of blocks, the first
  // partition's partial emitted where the second begins.
  int32_t pair_items;
  // Fused append (NULL append_slots: none): sequence s's new token, rows append_k/v + s * stride
  // (num_kv_heads * head_dim elements of q_dtype), goes to slot append_slots[s] (< 0: none), which
  // is the slot of position context_lens[s] - 1; the wavefront of each (s, KV head) row's last
  // item writes that head's part and takes the position from registers instead of the pool.
  const int64_t *append_slots;
  // With a shared prefix of append_from positions (0: none), a context of at most append_from
  // positions takes no write: its position lies in the shared blocks, which keep their bytes, and
  // the attention reads it from the pool.
  int32_t append_from;
  const void *append_k;
  const void *append_v;
  int64_t append_k_stride;
  int64_t append_v_stride;
  // Shared-prefix decode (0 / NULL for the plain decode): every sequence's first prefix_len
  // positions live in the blocks prefix_table[0 .. prefix_len / 16).  Workspace partition slots
  // 0 .. prefix_chunks - 1 of every row hold the prefix's chunks, the suffix partitions follow.
  const int32_t *prefix_table;
  int32_t prefix_len;       // multiple of 16
  int32_t prefix_chunks;    // ceil(prefix_len / kPrefixChunk)
  // Prefill (a chunk of new tokens per sequence): sequence s's tokens are query rows
  // query_start[s] .. query_start[s + 1] - 1, at positions context_lens[s] - n_s .. context_lens[s] - 1.
  const int32_t *query_start;
  int32_t max_query_len;    // host bound of query_start[s + 1] - query_start[s]
  // Dealing order of the persistent matrix-core grid (NULL: batch order): its item list runs over
  // sequences seq_order[0], seq_order[1], ...; an entry outside [0, num_seqs) is skipped.  Given
  // only while every per-sequence item count of the list stays below 2^kOrderCountBits.
  const int32_t *seq_order;
};

// The persistent grid keeps an ordered list's sequence ids beside the item counts in one LDS word.
constexpr int kOrderCountBits = 20;

// Whether a dealing order fits the list (at most `slots` items per sequence).
inline bool order_fits(int32_t num_seqs, int64_t slots) {
  return (int64_t)num_seqs * slots < ((int64_t)1 << kOrderCountBits);
}

// Partition `part` of positions [base, L) (base a multiple of the block size) cut into
// n = ceil((L - base) / PT) partitions: the range's nb blocks are shared out as evenly as whole
// blocks allow (the first nb mod n partitions take one block more), so no partition holds more than
// PT positions and the partitions of one range differ by at most one block.  Sets [*start, *end).
inline __host__ __device__ void partition_range(int32_t base, int32_t L, int32_t PT, int32_t part,
                                                int32_t *start, int32_t *end) {
  const int32_t len = L - base;
  const int32_t n = (len + PT - 1) / PT;
  const int32_t nb = (len + kBlock - 1) / kBlock;
  const int32_t q = nb / n, r = nb % n;
  const int32_t b0 = part * q + (part < r ? part : r);
  const int32_t b1 = b0 + q + (part < r ? 1 : 0);
  *start = base + b0 * kBlock;
  *end = base + b1 * kBlock < L ? base + b1 * kBlock : L;
}

// Workspace partition slots of a row whose context length is L (see DecodeArgs).
inline __host__ __device__ int32_t row_partitions(const DecodeArgs &a, int32_t L) {
  const int32_t PT = a.partition_size;
  if (a.prefix_len > 0)
    return a.prefix_chunks + (L > a.prefix_len ? (L - a.prefix_len + PT - 1) / PT : 0);
  return (L + PT - 1) / PT;
}

struct CopyArgs {
  static constexpr int kMaxLayers = 32;
  void *k_pools[kMaxLayers];
  void *v_pools[kMaxLayers];
  int32_t num_layers;
  int64_t block_bytes;  // bytes of one block in one pool (all KV heads)
  int32_t num_blocks;
  const int32_t *pairs;
  int32_t num_pairs;
};

struct SwapArgs {
  static constexpr int kMaxLayers = 32;
  void *dev_k[kMaxLayers];
  void *dev_v[kMaxLayers];
  void *host_k[kMaxLayers];  // device-side addresses of pinned host memory
  void *host_v[kMaxLayers];
  int32_t num_layers;
  int64_t block_bytes;  // bytes of one block in one pool (all KV heads)
  int32_t num_blocks;
  int32_t num_host;
  const int32_t *pairs;  // {device block, host slot}
  int32_t num_pairs;
  int32_t to_host;
};

// Fixed device scratch of pa_decode_attention_noalloc (scratch.hip): its size, and the current
// device's address of it (looked up once per device; no allocation).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void **ptr);

hipError_t launch_reshape_and_cache(const ReshapeArgs &a, hipStream_t stream);
hipError_t launch_swap_blocks(const SwapArgs &a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t stream);
bool decode_mfma_supports(const DecodeArgs &a);
bool decode_mfma_supports_prefix(const DecodeArgs &a);
// Wavefronts that take sequence items when the matrix-core kernel runs `a` on the current device
// (0: the direct grid, which deals no list).
int decode_mfma_item_waves(const DecodeArgs &a);
hipError_t launch_prefill_mfma(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_partition_reduce(const DecodeArgs &a, hipStream_t stream);

}  // namespace pa
