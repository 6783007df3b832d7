// pa_api.cpp — the C ABI of libpa.so (include/pa.h): argument validation, partition sizing and
// dispatch to the gfx950 kernels.  Nothing here allocates or synchronises device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_kernels.h"

namespace {

static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kNoAllocScratchBytes, "no-alloc scratch size");

thread_local std::string g_last_error;

pa_status fail(pa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() { return PA_OK; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool block_size_ok(int32_t b) { return b == 8 || b == PA_BLOCK_SIZE || b == 32; }

pa_status check_cache(const pa_cache *c, const char *who) {
  if (!c) return fail(PA_ERR_NULL, "%s: cache is NULL", who);
  if (!block_size_ok(c->block_size))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (8, 16 or 32 supported)", who,
                c->block_size);
  if (c->num_blocks < 0) return fail(PA_ERR_SHAPE, "%s: num_blocks %d < 0", who, c->num_blocks);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: num_kv_heads %d outside 1..16", who, c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128 supported)", who, c->head_dim);
  if (c->cache_dtype < PA_F32 || c->cache_dtype > PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: cache_dtype %d unknown", who, c->cache_dtype);
  if (!c->k_pool || !c->v_pool) return fail(PA_ERR_NULL, "%s: k_pool / v_pool is NULL", who);
  if (!aligned16(c->k_pool) || !aligned16(c->v_pool))
    return fail(PA_ERR_SHAPE, "%s: pools must be 16-byte aligned", who);
  const bool fp8 = c->cache_dtype == PA_FP8_E4M3;
  if (fp8 && (!c->k_scale || !c->v_scale))
    return fail(PA_ERR_NULL, "%s: an fp8 cache needs k_scale and v_scale", who);
  if (!fp8 && (c->k_scale || c->v_scale))
    return fail(PA_ERR_SHAPE, "%s: scales are only meaningful for an fp8 cache", who);
  return PA_OK;
}

pa::CacheArgs cache_args(const pa_cache *c) {
  pa::CacheArgs a;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.k_scale = c->k_scale;
  a.v_scale = c->v_scale;
  a.num_blocks = c->num_blocks;
  a.block_size = c->block_size;
  a.num_kv_heads = c->num_kv_heads;
  a.head_dim = c->head_dim;
  a.dtype = c->cache_dtype;
  return a;
}

pa_status launch_status(hipError_t e, const char *who) {
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s: %s", who, hipGetErrorString(e));
  return PA_OK;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Debug checks (PA_DEBUG): off unless the environment variable PA_DEBUG is set to a non-zero value
// when the library is first used, or pa_set_debug() turns them on.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char *e = std::getenv("PA_DEBUG");
    d = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, d, std::memory_order_relaxed);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d > 0;
}

// Debug mode only: n elements of a device (or pinned host) array, copied to the host once the
// stream has reached this point.
template <class T>
pa_status debug_fetch(const T *src, int64_t n, void *stream, std::vector<T> &dst, const char *who,
                      const char *what) {
  dst.assign((size_t)n, T());
  if (n == 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst.data(), src, (size_t)n * sizeof(T), hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(PA_ERR_LAUNCH, "%s: PA_DEBUG copy of %s failed: %s", who, what,
                hipGetErrorString(e));
  return PA_OK;
}

int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                          int32_t partition_size) {
  return partition_size > 0 ? partition_size
                            : pa_decode_auto_partition(num_seqs, num_kv_heads, max_context_len);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Partition slots per row for these sizes (plain decode: prefix_len = 0).
int64_t decode_slots(int32_t max_len, int32_t pt, int32_t prefix_len) {
  if (max_len <= 0) return 1;
  if (prefix_len <= 0) return ceil_div(max_len, pt);
  return ceil_div(prefix_len, pa::kPrefixChunk) +
         (max_len > prefix_len ? ceil_div(max_len - prefix_len, pt) : 0);
}

// Workspace: with more than one partition slot per row, or a shared prefix, the partials
// [S][Hq][slots][D] and their (m, l) [S][Hq][slots][2], fp32; none otherwise.
size_t partials_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int64_t slots) {
  const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)slots;
  return align256(rows * head_dim * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

size_t ws_bytes_for(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int64_t slots,
                    bool partials) {
  return partials ? partials_bytes(num_seqs, num_q_heads, head_dim, slots) : 0;
}


}  // namespace

extern "C" {

size_t pa_pool_bytes(const pa_cache *c) {
  if (!c || !block_size_ok(c->block_size) || c->num_blocks < 0 || c->num_kv_heads < 1 ||
      c->head_dim < 1)
    return 0;
  const int e = pa::dtype_bytes(c->cache_dtype);
  if (!e) return 0;
  return (size_t)c->num_blocks * c->num_kv_heads * c->block_size * c->head_dim * e;
}

pa_status pa_reshape_and_cache(const pa_cache *cache, const void *key, const void *value,
                               int32_t in_dtype, int64_t key_stride, int64_t value_stride,
                               const int64_t *slot_mapping, int32_t num_tokens, void *stream) {
  const char *who = "pa_reshape_and_cache";
  pa_status st = check_cache(cache, who);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "%s: num_tokens %d < 0", who, num_tokens);
  if (num_tokens == 0) return ok();
  if (!key || !value || !slot_mapping) return fail(PA_ERR_NULL, "%s: NULL key/value/slots", who);
  if (in_dtype < PA_F32 || in_dtype > PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: in_dtype %d (f32/f16/bf16 rows only)", who, in_dtype);
  if (cache->cache_dtype != PA_FP8_E4M3 && in_dtype != cache->cache_dtype)
    return fail(PA_ERR_UNSUPPORTED, "%s: rows of dtype %d into a cache of dtype %d", who, in_dtype,
                cache->cache_dtype);
  const int64_t row = (int64_t)cache->num_kv_heads * cache->head_dim;
  if (key_stride == 0) key_stride = row;
  if (value_stride == 0) value_stride = row;
  if (key_stride < row || value_stride < row)
    return fail(PA_ERR_SHAPE, "%s: strides %lld/%lld below a row of %lld elements", who,
                (long long)key_stride, (long long)value_stride, (long long)row);
  if (debug_on()) {
    std::vector<int64_t> h;
    st = debug_fetch(slot_mapping, num_tokens, stream, h, who, "slot_mapping");
    if (st != PA_OK) return st;
    st = pa_check_slots(h.data(), num_tokens, cache->num_blocks, cache->block_size);
    if (st != PA_OK) return fail(st, "%s: %s", who, g_last_error.c_str());
  }
  pa::ReshapeArgs a;
  a.cache = cache_args(cache);
  a.key = key;
  a.value = value;
  a.in_dtype = in_dtype;
  a.key_stride = key_stride;
  a.value_stride = value_stride;
  a.slots = slot_mapping;
  a.num_tokens = num_tokens;
  return launch_status(pa::launch_reshape_and_cache(a, static_cast<hipStream_t>(stream)), who);
}

int32_t pa_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  // Measured on MI355X: a few long (sequence, KV head) rows run best with 1,024-position
  // partitions (rare item prologues, still enough items to spread); many rows with long contexts
  // (two or more items per wavefront at any size) with 512 (fewer item boundaries per wavefront,
  // fewer partials); everything else with 256, halved (down to 64) while that leaves fewer than
  // 512 items to spread over the device.
  const int64_t rows = (int64_t)(num_seqs > 0 ? num_seqs : 1) * (num_kv_heads > 0 ? num_kv_heads : 1);
  const int32_t L = max_context_len > 0 ? max_context_len : 1;
  if (rows <= 64 && L >= 4096) return 1024;
  if (rows >= 2048 && L >= 8192) return 512;
  int32_t pt = 256;
  while (pt > 64 && rows * ceil_div(L, pt) < 512) pt /= 2;
  return pt;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  if (max_context_len <= 0) return 0;
  const int32_t pt = resolve_partition(num_seqs, num_kv_heads, max_context_len, partition_size);
  if (pt <= 0) return 0;
  const int64_t np = ceil_div(max_context_len, pt);
  return ws_bytes_for(num_seqs, num_q_heads, head_dim, np, np > 1);
}

}  // extern "C"

namespace {

// The appended tokens of pa_decode_attention_append: one row per sequence.
struct AppendIn {
  const void *key;
  const void *value;
  int64_t key_stride;
  int64_t value_stride;
  const int64_t *slots;
};

// Validation and dispatch shared by the plain and the shared-prefix decode, with or without the
// fused append.
// noalloc: the partials go to the library's fixed device scratch (pa_decode_attention_noalloc);
// workspace / workspace_bytes are then ignored.
pa_status decode_common(const char *who, void *out, const void *query, int32_t q_dtype,
                        int64_t q_stride, const pa_cache *cache, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *context_lens,
                        const int32_t *seq_order, int32_t num_seqs, int32_t num_q_heads,
                        int32_t max_context_len, float scale, const int32_t *prefix_table,
                        int32_t prefix_len, int32_t partition_size, void *workspace,
                        size_t workspace_bytes, uint32_t flags, void *stream,
                        const AppendIn *app = nullptr, bool noalloc = false) {
  pa_status st = check_cache(cache, who);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_SHAPE, "%s: num_seqs %d outside 0..65535", who, num_seqs);
  if (prefix_len < 0 || prefix_len % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "%s: prefix_len %d is not a non-negative multiple of 16", who,
                prefix_len);
  if (num_seqs == 0) return ok();
  if (!out || !query || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "%s: NULL out/query/block_tables/context_lens", who);
  if (prefix_len > 0 && !prefix_table) return fail(PA_ERR_NULL, "%s: NULL prefix_table", who);
  const int H = cache->num_kv_heads, D = cache->head_dim;
  if (num_q_heads < 1 || num_q_heads % H != 0)
    return fail(PA_ERR_SHAPE, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                num_q_heads, H);
  if (num_q_heads / H > 16)
    return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (at most 16)", who,
                num_q_heads / H);
  const int cdt = cache->cache_dtype;
  const bool combo_ok = (cdt == PA_FP8_E4M3) ? (q_dtype == PA_F16 || q_dtype == PA_BF16)
                                             : (q_dtype == cdt);
  if (!combo_ok)
    return fail(PA_ERR_UNSUPPORTED, "%s: query dtype %d with cache dtype %d", who, q_dtype, cdt);
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq %d < 1", who, max_blocks_per_seq);
  if (max_context_len < 0) return fail(PA_ERR_SHAPE, "%s: max_context_len < 0", who);
  if (partition_size < 0 || partition_size % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "%s: partition_size %d is not a non-negative multiple of 16", who,
                partition_size);
  if (q_stride == 0) q_stride = (int64_t)num_q_heads * D;
  if (q_stride < (int64_t)num_q_heads * D)
    return fail(PA_ERR_SHAPE, "%s: q_stride %lld below a row", who, (long long)q_stride);
  if ((flags & ~PA_DECODE_FORCE_VALU) != 0) return fail(PA_ERR_SHAPE, "%s: unknown flags", who);
  AppendIn ap{};
  if (app) {
    ap = *app;
    if (!ap.key || !ap.value || !ap.slots)
      return fail(PA_ERR_NULL, "%s: NULL key/value/slot_mapping", who);
    const int64_t row = (int64_t)H * D;
    if (ap.key_stride == 0) ap.key_stride = row;
    if (ap.value_stride == 0) ap.value_stride = row;
    if (ap.key_stride < row || ap.value_stride < row)
      return fail(PA_ERR_SHAPE, "%s: key/value strides %lld/%lld below a row of %lld elements",
                  who, (long long)ap.key_stride, (long long)ap.value_stride, (long long)row);
  }
  const int B = cache->block_size;
  if (B != PA_BLOCK_SIZE) {
    if (flags & PA_DECODE_FORCE_VALU)
      return fail(PA_ERR_UNSUPPORTED, "%s: the vector-ALU kernel needs block_size %d", who,
                  PA_BLOCK_SIZE);
    // 8-position blocks are read through one buffer descriptor per pool: 32-bit offsets
    if (B == 8 && pa_pool_bytes(cache) > (size_t)0xffff0000u)
      return fail(PA_ERR_UNSUPPORTED, "%s: block_size 8 needs a pool below 4 GiB", who);
  }

  if (debug_on()) {
    std::vector<int32_t> lens;
    st = debug_fetch(context_lens, num_seqs, stream, lens, who, "context_lens");
    if (st != PA_OK) return st;
    st = pa_check_context_lens(lens.data(), num_seqs, max_context_len);
    if (st != PA_OK) return fail(st, "%s: %s", who, g_last_error.c_str());
    if (app) {
      std::vector<int64_t> sl;
      st = debug_fetch(ap.slots, num_seqs, stream, sl, who, "slot_mapping");
      if (st != PA_OK) return st;
      st = pa_check_slots(sl.data(), num_seqs, cache->num_blocks, B);
      if (st != PA_OK) return fail(st, "%s: %s", who, g_last_error.c_str());
    }
    if (seq_order) {
      std::vector<int32_t> ord;
      st = debug_fetch(seq_order, num_seqs, stream, ord, who, "seq_order");
      if (st != PA_OK) return st;
      st = pa_check_seq_order(ord.data(), num_seqs);
      if (st != PA_OK) return fail(st, "%s: %s", who, g_last_error.c_str());
    }
  }
  const int64_t cap = (int64_t)max_blocks_per_seq * B;
  const int32_t max_len = (int32_t)(max_context_len < cap ? max_context_len : cap);
  pa::DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.q_stride = q_stride;
  a.q_dtype = q_dtype;
  a.cache = cache_args(cache);
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_context_len = max_len;
  a.scale = scale;
  a.persistent = 0;
  a.prefix_table = nullptr;
  a.prefix_len = 0;
  a.prefix_chunks = 0;
  a.partition_size = 0;
  a.num_partitions = 1;
  a.part_out = nullptr;
  a.part_ml = nullptr;
  a.seq_order = seq_order;
  const bool force_valu = (flags & PA_DECODE_FORCE_VALU) != 0;
  // The prefix's tiles need the matrix-core kernel on 16-position blocks; elsewhere the plain
  // decode gives the same result, each sequence reading the prefix through its own table.
  bool use_prefix = prefix_len > 0 && B == PA_BLOCK_SIZE;
  if (use_prefix) {
    pa::DecodeArgs t = a;
    t.prefix_len = prefix_len;
    use_prefix = !force_valu && pa::decode_mfma_supports_prefix(t);
  }
  // With a shared prefix only the kernel's own write keeps a context that ends inside the prefix
  // from being written (reshape_and_cache would write every slot): it needs 16-bit rows it can
  // read in pairs.
  if (app && prefix_len > 0 &&
      ((reinterpret_cast<uintptr_t>(ap.key) & 3u) != 0 ||
       (reinterpret_cast<uintptr_t>(ap.value) & 3u) != 0 || ap.key_stride % 2 != 0 ||
       ap.value_stride % 2 != 0))
    return fail(PA_ERR_SHAPE, "%s: with a shared prefix, key/value rows must be 4-byte aligned "
                "with even strides", who);
  // The automatic partition size follows the caller's max_context_len, as the workspace-size
  // functions do (the clamped max_len only bounds the number of partition slots).
  const int32_t pt = resolve_partition(
      num_seqs, H, use_prefix ? max_context_len - prefix_len : max_context_len, partition_size);
  const int64_t slots = decode_slots(max_len, pt, use_prefix ? prefix_len : 0);
  const bool partials = use_prefix || slots > 1;
  const size_t need = ws_bytes_for(num_seqs, num_q_heads, D, slots, partials);
  if (noalloc) {
    if (need > pa::kNoAllocScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "%s: the call needs %zu bytes of scratch, above the fixed %zu (use "
                  "pa_decode_attention with a workspace, or fewer sequences or a larger "
                  "partition_size)",
                  who, need, pa::kNoAllocScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const hipError_t e = pa::noalloc_scratch(&workspace);
      if (e != hipSuccess)
        return fail(PA_ERR_LAUNCH, "%s: device scratch lookup failed: %s", who,
                    hipGetErrorString(e));
      workspace_bytes = pa::kNoAllocScratchBytes;
    }
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                need);
  if (need > 0 && !aligned16(workspace))
    return fail(PA_ERR_SHAPE, "%s: workspace must be 16-byte aligned", who);
  a.partition_size = pt;
  a.num_partitions = (int32_t)slots;
  if (!pa::order_fits(num_seqs, slots)) a.seq_order = nullptr;
  if (use_prefix) {
    a.prefix_table = prefix_table;
    a.prefix_len = prefix_len;
    a.prefix_chunks = ceil_div(prefix_len, pa::kPrefixChunk);
  }
  if (partials) {
    char *ws = static_cast<char *>(workspace);
    const size_t rows = (size_t)num_seqs * num_q_heads * (size_t)slots;
    a.part_out = reinterpret_cast<float *>(ws);
    a.part_ml = reinterpret_cast<float *>(ws + align256(rows * D * sizeof(float)));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool use_mfma = use_prefix || (!force_valu && pa::decode_mfma_supports(a));
  // Every check runs before the first launch: a failed call enqueues nothing.
  if (!use_mfma && B != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: block_size %d runs on the matrix cores only (f16 or bf16 cache with the same "
                "query dtype, or fp8 cache with f16 queries; 16-byte aligned query rows, 8-byte "
                "aligned output)",
                who, B);
  // With a shared prefix, only the matrix-core kernel's own write keeps a context that ends inside
  // the prefix from writing its token into the shared blocks (the prefix kernel, or the plain
  // decode with append_from); the vector-ALU configurations are refused rather than appended by a
  // path without that guard.
  if (app && prefix_len > 0 && !use_mfma)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: the append with a shared prefix needs the matrix-core kernel (f16 / bf16 cache "
                "with the same query dtype or fp8 cache with f16 queries, no "
                "PA_DECODE_FORCE_VALU); call pa_reshape_and_cache and "
                "pa_decode_attention_shared_prefix instead",
                who);
  if (app) {
    // The matrix-core kernel writes the new tokens itself (16-bit rows read in pairs); elsewhere
    // reshape_and_cache runs first, with the same result.
    const bool fused = use_mfma && (reinterpret_cast<uintptr_t>(ap.key) & 3u) == 0 &&
                       (reinterpret_cast<uintptr_t>(ap.value) & 3u) == 0 &&
                       ap.key_stride % 2 == 0 && ap.value_stride % 2 == 0;
    if (fused) {
      a.append_slots = ap.slots;
      a.append_from = prefix_len;
      a.append_k = ap.key;
      a.append_v = ap.value;
      a.append_k_stride = ap.key_stride;
      a.append_v_stride = ap.value_stride;
    } else {
      pa::ReshapeArgs r;
      r.cache = a.cache;
      r.key = ap.key;
      r.value = ap.value;
      r.in_dtype = q_dtype;
      r.key_stride = ap.key_stride;
      r.value_stride = ap.value_stride;
      r.slots = ap.slots;
      r.num_tokens = num_seqs;
      const hipError_t er = pa::launch_reshape_and_cache(r, s);
      if (er != hipSuccess) return launch_status(er, who);
    }
  }
  // the matrix-core kernel keeps the partials of f16-query rows in fp16, with an fp8 cache in
  // units of the codes (the reduce applies the head's v_scale)
  a.part_f16 = use_mfma && q_dtype == PA_F16 ? 1 : 0;
  a.part_vscale = a.part_f16 && cdt == PA_FP8_E4M3 ? 1 : 0;
  hipError_t e = use_mfma ? pa::launch_decode_mfma(a, s) : pa::launch_decode_valu(a, s);
  if (e == hipSuccess) e = pa::launch_partition_reduce(a, s);
  return launch_status(e, who);
}

}  // namespace

extern "C" {

pa_status pa_decode_attention(void *out, const void *query, int32_t q_dtype, int64_t q_stride,
                              const pa_cache *cache, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              const int32_t *seq_order, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              void *workspace, size_t workspace_bytes, uint32_t flags,
                              void *stream) {
  return decode_common("pa_decode_attention", out, query, q_dtype, q_stride, cache, block_tables,
                       max_blocks_per_seq, context_lens, seq_order, num_seqs, num_q_heads,
                       max_context_len, scale, nullptr, 0, partition_size, workspace,
                       workspace_bytes, flags, stream);
}

pa_status pa_decode_attention_noalloc(void *out, const void *query, int32_t q_dtype,
                                      int64_t q_stride, const pa_cache *cache,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len, float scale,
                                      int32_t partition_size, uint32_t flags, void *stream) {
  return decode_common("pa_decode_attention_noalloc", out, query, q_dtype, q_stride, cache,
                       block_tables, max_blocks_per_seq, context_lens, nullptr, num_seqs,
                       num_q_heads, max_context_len, scale, nullptr, 0, partition_size, nullptr,
                       0, flags, stream, nullptr, true);
}

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
                                            uint32_t flags, void *stream) {
  return decode_common("pa_decode_attention_shared_prefix", out, query, q_dtype, q_stride, cache,
                       block_tables, max_blocks_per_seq, context_lens, seq_order, num_seqs,
                       num_q_heads, max_context_len, scale, prefix_table, prefix_len,
                       partition_size, workspace, workspace_bytes, flags, stream);
}

pa_status pa_decode_attention_append(void *out, const void *query, int32_t q_dtype,
                                     int64_t q_stride, const pa_cache *cache, const void *key,
                                     const void *value, int64_t key_stride, int64_t value_stride,
                                     const int64_t *slot_mapping, const int32_t *block_tables,
                                     int32_t max_blocks_per_seq, const int32_t *context_lens,
                                     const int32_t *seq_order, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_context_len, float scale,
                                     const int32_t *prefix_table, int32_t prefix_len,
                                     int32_t partition_size, void *workspace,
                                     size_t workspace_bytes, uint32_t flags, void *stream) {
  const AppendIn app{key, value, key_stride, value_stride, slot_mapping};
  return decode_common("pa_decode_attention_append", out, query, q_dtype, q_stride, cache,
                       block_tables, max_blocks_per_seq, context_lens, seq_order, num_seqs,
                       num_q_heads, max_context_len, scale, prefix_table, prefix_len,
                       partition_size, workspace, workspace_bytes, flags, stream, &app);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t prefix_len,
                                               int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || prefix_len < 0) return 0;
  if (prefix_len == 0)
    return pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                     max_context_len, partition_size);
  const int32_t ml = max_context_len > 0 ? max_context_len : 0;
  // enough for the prefix path and for the plain decode it falls back to
  const int32_t pt = resolve_partition(num_seqs, num_kv_heads, ml - prefix_len, partition_size);
  const size_t with_prefix = ws_bytes_for(num_seqs, num_q_heads, head_dim,
                                          decode_slots(ml, pt, prefix_len), true);
  const size_t plain = pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                 ml, partition_size);
  return with_prefix > plain ? with_prefix : plain;
}

pa_status pa_check_copy_pairs(const int32_t *pairs, int32_t num_pairs, int32_t num_blocks) {
  const char *who = "pa_check_copy_pairs";
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "%s: num_pairs < 0", who);
  if (num_pairs > 0 && !pairs) return fail(PA_ERR_NULL, "%s: pairs is NULL", who);
  if (num_blocks < 0) return fail(PA_ERR_SHAPE, "%s: num_blocks < 0", who);
  std::vector<char> is_dst((size_t)num_blocks, 0), is_src((size_t)num_blocks, 0);
  for (int32_t k = 0; k < num_pairs; ++k) {
    const int32_t s = pairs[2 * k], d = pairs[2 * k + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks)
      return fail(PA_ERR_SHAPE, "%s: pair %d = (%d, %d) outside the pool", who, k, s, d);
    is_src[(size_t)s] = 1;
  }
  for (int32_t k = 0; k < num_pairs; ++k) {
    const int32_t d = pairs[2 * k + 1];
    if (is_dst[(size_t)d]) return fail(PA_ERR_ALIAS, "%s: destination %d repeats", who, d);
    if (is_src[(size_t)d]) return fail(PA_ERR_ALIAS, "%s: destination %d is also a source", who, d);
    is_dst[(size_t)d] = 1;
  }
  return PA_OK;
}

pa_status pa_check_slots(const int64_t *slots, int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size) {
  const char *who = "pa_check_slots";
  if (num_tokens < 0 || num_blocks < 0 || block_size < 1)
    return fail(PA_ERR_SHAPE, "%s: negative count or block size", who);
  if (num_tokens > 0 && !slots) return fail(PA_ERR_NULL, "%s: slots is NULL", who);
  const int64_t n = (int64_t)num_blocks * block_size;
  std::vector<char> seen((size_t)n, 0);
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int64_t s = slots[t];
    if (s < 0 || s >= n) continue;  // skipped by the kernels
    if (seen[(size_t)s]) return fail(PA_ERR_ALIAS, "%s: slot %lld repeats (token %d)", who,
                                     (long long)s, t);
    seen[(size_t)s] = 1;
  }
  return PA_OK;
}

pa_status pa_check_context_lens(const int32_t *context_lens, int32_t num_seqs,
                                int32_t max_context_len) {
  const char *who = "pa_check_context_lens";
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "%s: num_seqs < 0", who);
  if (num_seqs > 0 && !context_lens) return fail(PA_ERR_NULL, "%s: context_lens is NULL", who);
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0)
      return fail(PA_ERR_SHAPE, "%s: context_lens[%d] = %d < 0", who, s, context_lens[s]);
    if (context_lens[s] > max_context_len)
      return fail(PA_ERR_SHAPE, "%s: context_lens[%d] = %d above max_context_len %d", who, s,
                  context_lens[s], max_context_len);
  }
  return PA_OK;
}

pa_status pa_check_seq_order(const int32_t *seq_order, int32_t num_seqs) {
  const char *who = "pa_check_seq_order";
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "%s: num_seqs < 0", who);
  if (num_seqs > 0 && !seq_order) return fail(PA_ERR_NULL, "%s: seq_order is NULL", who);
  std::vector<char> seen((size_t)num_seqs, 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t s = seq_order[i];
    if (s < 0 || s >= num_seqs)
      return fail(PA_ERR_SHAPE, "%s: seq_order[%d] = %d outside 0..%d", who, i, s, num_seqs - 1);
    if (seen[(size_t)s])
      return fail(PA_ERR_SHAPE, "%s: sequence %d appears twice (entry %d)", who, s, i);
    seen[(size_t)s] = 1;
  }
  return PA_OK;
}

namespace {

// Items of each sequence (partitions of pt positions after `base`, times the KV heads) and the
// 16-position steps of its largest item, as the kernel cuts them; returns the list's item count.
int64_t plan_items(const int32_t *context_lens, int32_t num_seqs, int32_t max_len, int32_t base,
                   bool use_prefix, int32_t pt, int H, std::vector<int32_t> &items,
                   std::vector<int32_t> &steps) {
  items.assign((size_t)num_seqs, 0);
  steps.assign((size_t)num_seqs, 0);
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = std::min(std::max(context_lens[s], 0), max_len);
    const int32_t n = L > base ? ceil_div(L - base, pt) : (use_prefix ? 0 : 1);
    items[(size_t)s] = n * H;
    steps[(size_t)s] = L > base ? ceil_div(ceil_div(L - base, pa::kBlock), n) : 0;
    total += items[(size_t)s];
  }
  return total;
}

// The dealing order of those items on `waves` item wavefronts (item f of the list goes to
// wavefront f mod waves), written to order[0 .. num_seqs); false, with the order untouched, where
// it has nothing to balance.
bool plan_arrange(const std::vector<int32_t> &items, const std::vector<int32_t> &steps,
                  int64_t total, int waves, bool use_prefix, int32_t *order) {
  const int32_t num_seqs = (int32_t)items.size();
  // Where no wavefront gets a second item and no prefix workgroups share the compute units
  // (whose third, late-starting workgroups the order feeds the small items), or where the list
  // fills at most half of one round, the order has nothing to balance and the ordered scan only
  // costs time (measured: 32 fp16 sequences of up to 2,048 positions, 608 items on 1,024
  // wavefronts, +0.3 us).
  if (2 * total <= waves || (total <= waves && !use_prefix)) return false;
  // The sequences by the steps of their largest item, largest first, ties in batch order: a
  // counting sort over the step counts (a stable comparison sort where they run very large).
  std::vector<int32_t> by_size((size_t)num_seqs);
  int32_t max_step = 0;
  for (int32_t s = 0; s < num_seqs; ++s) max_step = std::max(max_step, steps[(size_t)s]);
  if (max_step <= 8192) {
    std::vector<int32_t> start((size_t)max_step + 1, 0);
    for (int32_t s = 0; s < num_seqs; ++s) ++start[(size_t)steps[(size_t)s]];
    int32_t pos = 0;
    for (int32_t v = max_step; v >= 0; --v) {
      const int32_t c = start[(size_t)v];
      start[(size_t)v] = pos;
      pos += c;
    }
    for (int32_t s = 0; s < num_seqs; ++s) by_size[(size_t)start[(size_t)steps[(size_t)s]]++] = s;
  } else {
    for (int32_t s = 0; s < num_seqs; ++s) by_size[(size_t)s] = s;
    std::stable_sort(by_size.begin(), by_size.end(),
                     [&](int32_t x, int32_t y) { return steps[(size_t)x] > steps[(size_t)y]; });
  }
  int32_t k = 0;
  if (total > waves && total <= 2 * (int64_t)waves) {
    // Two rounds: total - waves wavefronts take two items, the others one.  The largest
    // sequences go to the one-item wavefronts (the last entries of the first round), the next
    // largest to the two-item wavefronts' first round, and the rest follow smallest first, so that
    // the second round gives the largest first-round items the smallest second ones.  A sequence
    // that does not fit a region goes to the next.
    const int64_t pairs = total - waves, singles = waves - pairs;
    std::vector<int32_t> first, single, second;
    int64_t nf = 0, ns = 0;
    for (int32_t s : by_size) {
      const int64_t n = items[(size_t)s];
      if (ns + n <= singles) {
        single.push_back(s);
        ns += n;
      } else if (nf + n <= pairs) {
        first.push_back(s);
        nf += n;
      } else {
        second.push_back(s);
      }
    }
    for (int32_t s : first) order[k++] = s;
    for (int32_t s : single) order[k++] = s;
    for (auto it = second.rbegin(); it != second.rend(); ++it) order[k++] = *it;
  } else {
    // Rounds of `waves` items, filled alternately with the largest and the smallest items left,
    // so that a wavefront given a large item in one round is given a small one in the next.
    int32_t lo = 0, hi = num_seqs - 1;
    for (int round = 0; lo <= hi; ++round) {
      int64_t n = 0;
      while (lo <= hi && n < waves) {
        const int32_t s = (round % 2 == 0) ? by_size[(size_t)lo++] : by_size[(size_t)hi--];
        order[k++] = s;
        n += items[(size_t)s];
      }
    }
  }
  return true;
}

// 16-position steps of the busiest wavefront when order's list is dealt item f -> wavefront
// f mod waves, every item of a sequence counted at its largest item's steps.  A sequence's items
// are a run of the list, so each adds its steps to a cyclic range of wavefronts (a difference
// array: O(num_seqs + waves)).
int64_t busiest_steps(const int32_t *order, const std::vector<int32_t> &items,
                      const std::vector<int32_t> &steps, int waves) {
  std::vector<int64_t> diff((size_t)waves + 1, 0);
  int64_t every = 0, f = 0;
  for (size_t k = 0; k < items.size(); ++k) {
    const int32_t s = order[k];
    const int64_t n = items[(size_t)s], v = steps[(size_t)s];
    if (n == 0) continue;
    every += (n / waves) * v;
    const int64_t r = n % waves, w0 = f % waves;
    if (r > 0) {
      diff[(size_t)w0] += v;
      if (w0 + r <= waves) {
        diff[(size_t)(w0 + r)] -= v;
      } else {
        diff[(size_t)waves] -= v;
        diff[0] += v;
        diff[(size_t)(w0 + r - waves)] -= v;
      }
    }
    f += n;
  }
  int64_t run = 0, best = 0;
  for (int w = 0; w < waves; ++w) {
    run += diff[(size_t)w];
    best = std::max(best, run);
  }
  return every + best;
}

// Planned partition sizes: multiples of this step above the automatic size, up to the last.
constexpr int32_t kPlanPartitionStep = 64;
constexpr int32_t kPlanPartitionMax = 2048;
// What one more round of items costs, in bytes of the busiest wavefront's KV stream.
constexpr double kPlanRoundBytes = 240.0 * 1024.0;

}  // namespace

pa_status pa_decode_plan(const pa_cache *cache, int32_t q_dtype, const int32_t *context_lens,
                         int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                         int32_t max_context_len, int32_t prefix_len, int32_t partition_size,
                         uint32_t flags, int32_t *seq_order, int32_t *round_items,
                         int32_t *partition_size_out) {
  const char *who = "pa_decode_plan";
  pa_status st = check_cache(cache, who);
  if (st != PA_OK) return st;
  if (round_items) *round_items = 0;
  if (partition_size_out) *partition_size_out = partition_size;
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_SHAPE, "%s: num_seqs %d outside 0..65535", who, num_seqs);
  if (num_seqs == 0) return ok();
  if (!context_lens || !seq_order) return fail(PA_ERR_NULL, "%s: NULL context_lens/seq_order", who);
  const int H = cache->num_kv_heads, B = cache->block_size;
  if (num_q_heads < 1 || num_q_heads % H != 0)
    return fail(PA_ERR_SHAPE, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                num_q_heads, H);
  if (max_blocks_per_seq < 1 || max_context_len < 0 || prefix_len < 0 ||
      prefix_len % PA_BLOCK_SIZE != 0 || partition_size < 0 || partition_size % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_SHAPE, "%s: bad max_blocks_per_seq / max_context_len / prefix_len / "
                "partition_size", who);
  if ((flags & ~(PA_DECODE_FORCE_VALU | PA_DECODE_PLAN_APPEND)) != 0)
    return fail(PA_ERR_SHAPE, "%s: unknown flags", who);
  for (int32_t s = 0; s < num_seqs; ++s) seq_order[s] = s;

  // The kernel and grid the decode call would use (the checks of decode_common that choose them).
  const int64_t cap = (int64_t)max_blocks_per_seq * B;
  const int32_t max_len = (int32_t)(max_context_len < cap ? max_context_len : cap);
  const bool force_valu = (flags & PA_DECODE_FORCE_VALU) != 0;
  static const int64_t kAnySlot = 0;
  pa::DecodeArgs a{};
  a.q_dtype = q_dtype;
  a.cache = cache_args(cache);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_context_len = max_len;
  a.append_slots = (flags & PA_DECODE_PLAN_APPEND) ? &kAnySlot : nullptr;
  bool use_prefix = prefix_len > 0 && B == PA_BLOCK_SIZE;
  if (use_prefix) {
    pa::DecodeArgs t = a;
    t.prefix_len = prefix_len;
    use_prefix = !force_valu && pa::decode_mfma_supports_prefix(t);
  }
  const bool use_mfma = use_prefix || (!force_valu && pa::decode_mfma_supports(a));
  if (!use_mfma) return ok();  // the vector-ALU kernel deals no list
  const int32_t base = use_prefix ? prefix_len : 0;
  // The list and grid at partition size pt: the call's partition slots, its item wavefronts (0:
  // the direct grid, or an order the call would ignore) and the items.
  std::vector<int32_t> items, steps;
  auto setup = [&](int32_t pt, int64_t *total) {
    a.partition_size = pt;
    a.num_partitions = (int32_t)decode_slots(max_len, pt, base);
    if (use_prefix) {
      a.prefix_len = prefix_len;
      a.prefix_chunks = ceil_div(prefix_len, pa::kPrefixChunk);
    }
    if (!pa::order_fits(num_seqs, a.num_partitions)) return 0;
    const int waves = pa::decode_mfma_item_waves(a);
    if (waves > 0)
      *total = plan_items(context_lens, num_seqs, max_len, base, use_prefix, pt, H, items, steps);
    return waves;
  };
  const int32_t pt0 = resolve_partition(num_seqs, H, max_context_len - base, partition_size);
  int32_t pt = pt0;
  int64_t total = 0;
  int waves = setup(pt0, &total);
  if (waves <= 0) return ok();
  // Automatic partitions of a plain decode whose list takes more than one round: larger
  // partitions mean fewer items, each of which costs its wavefront a ring fill and drain, a
  // partial and a merge, but a longer busiest wavefront.  Each candidate size's list is arranged
  // and dealt as below, and the size with the least (busiest wavefront's KV bytes + one round's
  // cost per round of items) is kept; sizes whose list fits one round are not taken (the deal then
  // has nothing to balance: the fp8 batch of 512 sequences took 129 us on 3,008 items against
  // 107 us on 3,720).  Only sizes above the automatic one are tried, so a workspace sized for it
  // still serves the call.
  if (partition_size == 0 && !use_prefix && total > waves) {
    const int eb = a.cache.dtype == pa::kFP8 ? 1 : (a.cache.dtype == pa::kF32 ? 4 : 2);
    const double step_bytes = 2.0 * pa::kBlock * a.cache.head_dim * eb;
    std::vector<int32_t> trial((size_t)num_seqs);
    double best = -1.0;
    for (int32_t c = pt0; c <= std::max(pt0, kPlanPartitionMax); c += kPlanPartitionStep) {
      int64_t tc = 0;
      const int wc = setup(c, &tc);
      if (wc <= 0 || tc <= wc) break;
      for (int32_t s = 0; s < num_seqs; ++s) trial[(size_t)s] = s;
      plan_arrange(items, steps, tc, wc, false, trial.data());
      const double cost = (double)busiest_steps(trial.data(), items, steps, wc) * step_bytes +
                          kPlanRoundBytes * (double)tc / wc;
      if (best < 0.0 || cost < best) {
        best = cost;
        pt = c;
      }
    }
    waves = setup(pt, &total);
    if (pt != pt0 && partition_size_out) *partition_size_out = pt;
  }
  if (!plan_arrange(items, steps, total, waves, use_prefix, seq_order)) return ok();
  if (round_items) *round_items = waves;
  return ok();
}

void pa_set_debug(int on) { g_debug.store(on ? 1 : 0, std::memory_order_relaxed); }

int pa_debug_enabled(void) { return debug_on() ? 1 : 0; }

pa_status pa_copy_blocks(const pa_cache *layers, int32_t num_layers, const int32_t *block_pairs,
                         int32_t num_pairs, void *stream) {
  const char *who = "pa_copy_blocks";
  if (num_layers < 0 || num_pairs < 0) return fail(PA_ERR_SHAPE, "%s: negative count", who);
  if (num_layers == 0 || num_pairs == 0) return ok();
  if (!layers || !block_pairs) return fail(PA_ERR_NULL, "%s: NULL layers / block_pairs", who);
  for (int32_t l = 0; l < num_layers; ++l) {
    pa_status st = check_cache(&layers[l], who);
    if (st != PA_OK) return st;
    if (layers[l].num_blocks != layers[0].num_blocks ||
        layers[l].block_size != layers[0].block_size ||
        layers[l].num_kv_heads != layers[0].num_kv_heads ||
        layers[l].head_dim != layers[0].head_dim || layers[l].cache_dtype != layers[0].cache_dtype)
      return fail(PA_ERR_SHAPE, "%s: layer %d differs in shape or dtype from layer 0", who, l);
  }
  if (debug_on()) {
    std::vector<int32_t> h;
    pa_status st = debug_fetch(block_pairs, 2 * (int64_t)num_pairs, stream, h, who, "block_pairs");
    if (st != PA_OK) return st;
    st = pa_check_copy_pairs(h.data(), num_pairs, layers[0].num_blocks);
    if (st != PA_OK) return fail(st, "%s: %s", who, g_last_error.c_str());
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t block_bytes = (int64_t)layers[0].num_kv_heads * layers[0].block_size *
                              layers[0].head_dim * pa::dtype_bytes(layers[0].cache_dtype);
  for (int32_t l0 = 0; l0 < num_layers; l0 += pa::CopyArgs::kMaxLayers) {
    pa::CopyArgs a;
    a.num_layers = num_layers - l0 < pa::CopyArgs::kMaxLayers ? num_layers - l0
                                                              : pa::CopyArgs::kMaxLayers;
    for (int32_t l = 0; l < a.num_layers; ++l) {
      a.k_pools[l] = layers[l0 + l].k_pool;
      a.v_pools[l] = layers[l0 + l].v_pool;
    }
    a.block_bytes = block_bytes;
    a.num_blocks = layers[0].num_blocks;
    a.pairs = block_pairs;
    a.num_pairs = num_pairs;
    pa_status st = launch_status(pa::launch_copy_blocks(a, s), who);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

pa_status pa_prefill_attention(void *out, const void *query, int32_t q_dtype, int64_t q_stride,
                               const pa_cache *cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               const int32_t *query_start, int32_t num_seqs, int32_t num_tokens,
                               int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                               float scale, void *stream) {
  const char *who = "pa_prefill_attention";
  pa_status st = check_cache(cache, who);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_SHAPE, "%s: num_seqs %d outside 0..65535", who, num_seqs);
  if (num_tokens < 0 || max_query_len < 0 || max_context_len < 0)
    return fail(PA_ERR_SHAPE, "%s: negative num_tokens / max_query_len / max_context_len", who);
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return ok();
  if (!out || !query || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_NULL, "%s: NULL out/query/block_tables/context_lens/query_start", who);
  const int H = cache->num_kv_heads, D = cache->head_dim;
  if (num_q_heads < 1 || num_q_heads % H != 0)
    return fail(PA_ERR_SHAPE, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                num_q_heads, H);
  if (max_blocks_per_seq < 1)
    return fail(PA_ERR_SHAPE, "%s: max_blocks_per_seq %d < 1", who, max_blocks_per_seq);
  if (q_stride == 0) q_stride = (int64_t)num_q_heads * D;
  if (q_stride < (int64_t)num_q_heads * D)
    return fail(PA_ERR_SHAPE, "%s: q_stride %lld below a row", who, (long long)q_stride);
  const int64_t groups = ((int64_t)max_query_len * (num_q_heads / H) + 63) / 64;
  if ((int64_t)num_seqs * H * groups > 0x7fffffff)
    return fail(PA_ERR_SHAPE, "%s: grid of %lld workgroups too large", who,
                (long long)((int64_t)num_seqs * H * groups));
  if (cache->block_size != PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "%s: prefill needs block_size %d", who, PA_BLOCK_SIZE);
  const int64_t cap = (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE;
  pa::DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.q_stride = q_stride;
  a.q_dtype = q_dtype;
  a.cache = cache_args(cache);
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_context_len = (int32_t)(max_context_len < cap ? max_context_len : cap);
  a.scale = scale;
  a.partition_size = 0;
  a.num_partitions = 1;
  a.query_start = query_start;
  a.max_query_len = max_query_len;
  if (!pa::decode_mfma_supports(a))
    return fail(PA_ERR_UNSUPPORTED,
                "%s: prefill runs on the matrix cores only (f16 or bf16 cache with the same query "
                "dtype, or fp8 cache with f16 queries; head_dim 64 or 128; at most 16 query heads "
                "per KV head; 16-byte aligned query rows, 8-byte aligned output; a non-empty pool)",
                who);
  return launch_status(pa::launch_prefill_mfma(a, static_cast<hipStream_t>(stream)), who);
}

// The device-side address of memory the GPU can reach: device memory, or pinned host memory
// (hipHostMalloc).  Pageable host memory, or a pointer HIP does not know, gives nullptr.
static void *device_reachable(const void *p, bool host_only) {
  hipPointerAttribute_t attr;
  if (!p || hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return nullptr;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer) return attr.devicePointer;
  if (!host_only && attr.type == hipMemoryTypeDevice) return const_cast<void *>(p);
  return nullptr;
}

pa_status pa_swap_blocks(const pa_cache *layers, int32_t num_layers, void *const *host_k,
                         void *const *host_v, int32_t num_host_blocks, const int32_t *block_pairs,
                         int32_t num_pairs, int32_t to_host, void *stream) {
  const char *who = "pa_swap_blocks";
  if (num_layers < 0 || num_pairs < 0 || num_host_blocks < 0)
    return fail(PA_ERR_SHAPE, "%s: negative count", who);
  if (num_layers == 0 || num_pairs == 0) return ok();
  if (!layers || !host_k || !host_v || !block_pairs)
    return fail(PA_ERR_NULL, "%s: NULL layers / host pools / block_pairs", who);
  for (int32_t l = 0; l < num_layers; ++l) {
    pa_status st = check_cache(&layers[l], who);
    if (st != PA_OK) return st;
    if (layers[l].num_blocks != layers[0].num_blocks ||
        layers[l].block_size != layers[0].block_size ||
        layers[l].num_kv_heads != layers[0].num_kv_heads ||
        layers[l].head_dim != layers[0].head_dim || layers[l].cache_dtype != layers[0].cache_dtype)
      return fail(PA_ERR_SHAPE, "%s: layer %d differs in shape or dtype from layer 0", who, l);
    if (!host_k[l] || !host_v[l]) return fail(PA_ERR_NULL, "%s: NULL host pool, layer %d", who, l);
  }
  const int32_t *pairs = static_cast<const int32_t *>(device_reachable(block_pairs, false));
  if (!pairs)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: block_pairs is neither device memory nor pinned host memory", who);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t block_bytes = (int64_t)layers[0].num_kv_heads * layers[0].block_size *
                              layers[0].head_dim * pa::dtype_bytes(layers[0].cache_dtype);
  for (int32_t l0 = 0; l0 < num_layers; l0 += pa::SwapArgs::kMaxLayers) {
    pa::SwapArgs a;
    a.num_layers = num_layers - l0 < pa::SwapArgs::kMaxLayers ? num_layers - l0
                                                              : pa::SwapArgs::kMaxLayers;
    for (int32_t l = 0; l < a.num_layers; ++l) {
      a.dev_k[l] = layers[l0 + l].k_pool;
      a.dev_v[l] = layers[l0 + l].v_pool;
      a.host_k[l] = device_reachable(host_k[l0 + l], true);
      a.host_v[l] = device_reachable(host_v[l0 + l], true);
      if (!a.host_k[l] || !a.host_v[l])
        return fail(PA_ERR_UNSUPPORTED,
                    "%s: host pool of layer %d is not pinned host memory the device can reach", who,
                    l0 + l);
    }
    a.block_bytes = block_bytes;
    a.num_blocks = layers[0].num_blocks;
    a.num_host = num_host_blocks;
    a.pairs = pairs;
    a.num_pairs = num_pairs;
    a.to_host = to_host != 0;
    pa_status st = launch_status(pa::launch_swap_blocks(a, s), who);
    if (st != PA_OK) return st;
  }
  return PA_OK;
}

const char *pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "bad shape or size";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_ALIAS: return "overlapping copy pairs";
    case PA_ERR_LAUNCH: return "kernel launch failed";
    case PA_ERR_NO_BLOCKS: return "no free blocks";
    case PA_ERR_STATE: return "bad sequence or block id";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
