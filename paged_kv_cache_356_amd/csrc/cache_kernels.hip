// cache_kernels.hip — reshape_and_cache (write each new token's K/V into its slot) and
// copy_blocks (the clone step of copy-on-write) for gfx950.
//
// reshape_and_cache: a generated token's K and V land in the next unused slot of its sequence's
// last block ("LLM Inference Visualizer, Lesson 06", "How paging grows"), where every later token
// reads them ("PagedAttention, Visualized", Part 2).
// copy_blocks: a writer into a shared block gets a clone of that one block ("PagedAttention"
// (devoured.fyi), "Copy-on-write: when two requests share a prefix").
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

// One workgroup per token.  16-bit caches: thread v handles K vector c (E elements of head h) of
// that token, writing the 16-byte K vector in one store and the E transposed V elements one by one.
// fp8 caches: thread v handles 4 elements (one 4-byte word of a K vector), so that all 128 threads
// share the token's divisions and encodings instead of 32 of them doing 16 each.
template <class CT, class IT>
__global__ __launch_bounds__(128) void reshape_and_cache_kernel(ReshapeArgs a) {
  const int t = blockIdx.x;
  const int64_t slot = a.slots[t];
  const CacheArgs &c = a.cache;
  const int B = c.block_size;
  if (slot < 0 || slot >= (int64_t)c.num_blocks * B) return;  // padding / out of range
  const int64_t blk = slot / B;
  const int off = (int)(slot % B);
  const int H = c.num_kv_heads, D = c.head_dim;
  using L = Layout<CT::bytes>;
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr int E = L::E;
  constexpr int P = kFP8 ? 4 : E;  // elements per thread
  const int per_head = D / P;
  const auto *key = static_cast<const typename IT::raw *>(a.key) + (size_t)t * a.key_stride;
  const auto *val = static_cast<const typename IT::raw *>(a.value) + (size_t)t * a.value_stride;
  auto *kp = static_cast<typename CT::raw *>(c.k_pool);
  auto *vp = static_cast<typename CT::raw *>(c.v_pool);
  for (int v = threadIdx.x; v < H * per_head; v += blockDim.x) {
    const int h = v / per_head;
    const int i0 = (v % per_head) * P;
    const size_t tile = L::tile(blk, h, H, D, B);
    if constexpr (kFP8) {
      const float ks = c.k_scale[h], vs = c.v_scale[h];
      uint32_t kw = 0;
      uint8_t ve[P];
#pragma unroll
      for (int j = 0; j < P; ++j) {
        kw |= (uint32_t)f32_to_e4m3(__fdiv_rn(load_f32<IT>(key, (size_t)h * D + i0 + j), ks))
              << (8 * j);
        ve[j] = f32_to_e4m3(__fdiv_rn(load_f32<IT>(val, (size_t)h * D + i0 + j), vs));
      }
      // K: the 4 elements are one aligned word of a 16-byte vector of the tile.
      *reinterpret_cast<uint32_t *>(kp + tile + L::k_off(off, i0, B)) = kw;
      // V: transposed tile, element (off, i) at i * B + off.
#pragma unroll
      for (int j = 0; j < P; ++j) vp[tile + L::v_off(off, i0 + j, B)] = ve[j];
    } else {
      static_assert(std::is_same<CT, IT>::value, "non-fp8 caches take rows of their own dtype");
      union {
        uint4 v;
        typename CT::raw e[E];
      } kv, vv;
#pragma unroll
      for (int j = 0; j < E; ++j) {  // same dtype: bit copy
        kv.e[j] = key[(size_t)h * D + i0 + j];
        vv.e[j] = val[(size_t)h * D + i0 + j];
      }
      // K: the E elements are one contiguous 16-byte vector of the tile.
      *reinterpret_cast<uint4 *>(kp + tile + L::k_off(off, i0, B)) = kv.v;
      // V: transposed tile, element (off, i) at i * B + off.
#pragma unroll
      for (int j = 0; j < E; ++j) vp[tile + L::v_off(off, i0 + j, B)] = vv.e[j];
    }
  }
}

template <class CT, class IT>
hipError_t reshape_launch(const ReshapeArgs &a, hipStream_t s) {
  reshape_and_cache_kernel<CT, IT><<<dim3(a.num_tokens), dim3(128), 0, s>>>(a);
  return hipGetLastError();
}

// One workgroup per (pair, layer, chunk of 64 KiB of the block's span in both pools).  Every
// thread issues all of its 16-byte loads before its first store (the source and destination blocks
// are distinct, which the restrict qualifiers state), so a copy costs one memory round trip.
constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;  // 16-byte vectors per thread and pool in one chunk (16 KiB)
constexpr int64_t kCopyChunk = (int64_t)kCopyThreads * kCopyVecs;  // vectors per chunk and pool

// The argument struct of a kernel as it sits in the kernel-argument segment.  Indexing its
// per-layer pointer arrays with the (wave-uniform) layer through this pointer reads them with
// scalar loads; indexing the by-value parameter would first copy the whole struct to per-lane
// scratch memory.  The struct is the kernel's only parameter, at offset 0.
template <class Args>
__device__ __forceinline__ const __attribute__((address_space(4))) Args *kernel_args() {
  return (const __attribute__((address_space(4))) Args *)__builtin_amdgcn_kernarg_segment_ptr();
}

// Whole blocks from src to dst, one chunk of kCopyChunk 16-byte vectors per pool and workgroup:
// every load of the chunk is issued before any store.  Loads past the block's end re-read its last
// vector (always in bounds) and are not stored, so the staging registers are written on every path
// and stay in registers.
__device__ __forceinline__ void copy_chunk(const uint4 *__restrict__ ks, const uint4 *__restrict__ vs,
                                           uint4 *__restrict__ kd, uint4 *__restrict__ vd,
                                           int64_t nvec) {
  const int64_t v0 = (int64_t)blockIdx.z * kCopyChunk;
  uint4 kx[kCopyVecs], vx[kCopyVecs];
#pragma unroll
  for (int k = 0; k < kCopyVecs; ++k) {
    const int64_t i = v0 + threadIdx.x + (int64_t)k * kCopyThreads;
    const int64_t j = i < nvec ? i : nvec - 1;
    kx[k] = ks[j];
    vx[k] = vs[j];
  }
#pragma unroll
  for (int k = 0; k < kCopyVecs; ++k) {
    const int64_t i = v0 + threadIdx.x + (int64_t)k * kCopyThreads;
    if (i < nvec) {
      kd[i] = kx[k];
      vd[i] = vx[k];
    }
  }
}

// Swapping: for pair p = {device block d, host slot h} and layer blockIdx.y, both pools' block d
// to slot h of the pinned host pools (to_host) or back.
__global__ __launch_bounds__(kCopyThreads) void swap_blocks_kernel(SwapArgs) {
  const auto *a = kernel_args<SwapArgs>();
  const int p = blockIdx.x, layer = blockIdx.y;
  const int d = a->pairs[2 * p], h = a->pairs[2 * p + 1];
  if (d < 0 || d >= a->num_blocks || h < 0 || h >= a->num_host) return;
  const int64_t bb = a->block_bytes;
  char *dk = static_cast<char *>(a->dev_k[layer]) + (size_t)d * bb;
  char *dv = static_cast<char *>(a->dev_v[layer]) + (size_t)d * bb;
  char *hk = static_cast<char *>(a->host_k[layer]) + (size_t)h * bb;
  char *hv = static_cast<char *>(a->host_v[layer]) + (size_t)h * bb;
  if (a->to_host)
    copy_chunk(reinterpret_cast<const uint4 *>(dk), reinterpret_cast<const uint4 *>(dv),
               reinterpret_cast<uint4 *>(hk), reinterpret_cast<uint4 *>(hv), bb / 16);
  else
    copy_chunk(reinterpret_cast<const uint4 *>(hk), reinterpret_cast<const uint4 *>(hv),
               reinterpret_cast<uint4 *>(dk), reinterpret_cast<uint4 *>(dv), bb / 16);
}

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs) {
  const auto *ap = kernel_args<CopyArgs>();
  const auto &a = *ap;
  const int p = blockIdx.x, layer = blockIdx.y;
  const int src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
  if (src < 0 || src >= a.num_blocks || dst < 0 || dst >= a.num_blocks) return;
  const uint4 *ks = reinterpret_cast<const uint4 *>(static_cast<const char *>(a.k_pools[layer]) +
                                                    (size_t)src * a.block_bytes);
  const uint4 *vs = reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v_pools[layer]) +
                                                    (size_t)src * a.block_bytes);
  uint4 *kd = reinterpret_cast<uint4 *>(static_cast<char *>(a.k_pools[layer]) +
                                        (size_t)dst * a.block_bytes);
  uint4 *vd = reinterpret_cast<uint4 *>(static_cast<char *>(a.v_pools[layer]) +
                                        (size_t)dst * a.block_bytes);
  copy_chunk(ks, vs, kd, vd, a.block_bytes / 16);
}

}  // namespace

hipError_t launch_reshape_and_cache(const ReshapeArgs &a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  switch (a.cache.dtype) {
    case kF32: return reshape_launch<f32_t, f32_t>(a, s);
    case kF16: return reshape_launch<f16_t, f16_t>(a, s);
    case kBF16: return reshape_launch<bf16_t, bf16_t>(a, s);
    case kFP8:
      switch (a.in_dtype) {
        case kF32: return reshape_launch<fp8_t, f32_t>(a, s);
        case kF16: return reshape_launch<fp8_t, f16_t>(a, s);
        case kBF16: return reshape_launch<fp8_t, bf16_t>(a, s);
        default: return hipErrorInvalidValue;
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_swap_blocks(const SwapArgs &a, hipStream_t s) {
  if (a.num_pairs == 0 || a.num_layers == 0) return hipSuccess;
  const int64_t nvec = a.block_bytes / 16;
  const unsigned chunks = (unsigned)((nvec + kCopyChunk - 1) / kCopyChunk);
  swap_blocks_kernel<<<dim3(a.num_pairs, a.num_layers, chunks), dim3(kCopyThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs &a, hipStream_t s) {
  if (a.num_pairs == 0 || a.num_layers == 0) return hipSuccess;
  const int64_t nvec = a.block_bytes / 16;
  const unsigned chunks = (unsigned)((nvec + kCopyChunk - 1) / kCopyChunk);
  copy_blocks_kernel<<<dim3(a.num_pairs, a.num_layers, chunks), dim3(kCopyThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace pa
