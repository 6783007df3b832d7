// calibrate.hip — the read-bandwidth reference: read the listed K/V tiles of two pools and nothing
// else (no products, no softmax, no stores beyond one word per workgroup), so that the decode
// kernels' achieved bandwidth can be set against a plain read of the same bytes on this device.
//
// One wavefront per list entry: it issues every 16-byte load of the entry's K tile and V tile at
// once (tile_bytes / 512 loads per lane, a whole 1 KiB per wave-wide load, with the non-temporal
// hint the decode kernels use), then folds them into one word.  The grid holds one workgroup per
// four entries and the hardware keeps as many of them in flight as fit on the device.
#include <hip/hip_runtime.h>

#include "pa_calibrate.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct CalArgs {
  const char *k_pool, *v_pool;
  int64_t tile_bytes;
  const int32_t *tiles;
  int64_t num_tiles;
  uint32_t *sink;
};

// kC: 1 KiB chunks per tile (1, 2, 4 or 8), or 0 for any other size (a loop over the chunks).
template <int kC>
__global__ __launch_bounds__(256) void calibrate_read_kernel(CalArgs a) {
  __shared__ uint32_t part[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t e = (int64_t)blockIdx.x * 4 + w;
  uint32_t acc = 0;
  if (e < a.num_tiles) {
    const int64_t t = a.tiles ? a.tiles[e] : e;
    const u32x4_t *k = reinterpret_cast<const u32x4_t *>(a.k_pool + t * a.tile_bytes) + lane;
    const u32x4_t *v = reinterpret_cast<const u32x4_t *>(a.v_pool + t * a.tile_bytes) + lane;
    if constexpr (kC > 0) {
      u32x4_t x[2 * kC];
#pragma unroll
      for (int i = 0; i < kC; ++i) x[i] = __builtin_nontemporal_load(k + 64 * i);
#pragma unroll
      for (int i = 0; i < kC; ++i) x[kC + i] = __builtin_nontemporal_load(v + 64 * i);
#pragma unroll
      for (int i = 0; i < 2 * kC; ++i) acc ^= x[i].x ^ x[i].y ^ x[i].z ^ x[i].w;
    } else {
      const int64_t c = a.tile_bytes >> 10;
      for (int64_t i = 0; i < c; ++i) {
        const u32x4_t y = __builtin_nontemporal_load(k + 64 * i);
        const u32x4_t z = __builtin_nontemporal_load(v + 64 * i);
        acc ^= y.x ^ y.y ^ y.z ^ y.w ^ z.x ^ z.y ^ z.z ^ z.w;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) part[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) a.sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" pa_status pa_calibrate_read(const void *k_pool, const void *v_pool, int64_t tile_bytes,
                                       const int32_t *tiles, int64_t num_tiles, uint32_t *sink,
                                       void *stream) {
  if (!k_pool || !v_pool || !sink) return PA_ERR_NULL;
  if (tile_bytes <= 0 || tile_bytes % 1024 != 0 || num_tiles < 0 || num_tiles > (1ll << 33))
    return PA_ERR_SHAPE;
  if (num_tiles == 0) return PA_OK;
  CalArgs a;
  a.k_pool = static_cast<const char *>(k_pool);
  a.v_pool = static_cast<const char *>(v_pool);
  a.tile_bytes = tile_bytes;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.sink = sink;
  const dim3 grid((unsigned)((num_tiles + 3) / 4)), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (tile_bytes >> 10) {
    case 1: calibrate_read_kernel<1><<<grid, block, 0, s>>>(a); break;
    case 2: calibrate_read_kernel<2><<<grid, block, 0, s>>>(a); break;
    case 4: calibrate_read_kernel<4><<<grid, block, 0, s>>>(a); break;
    case 8: calibrate_read_kernel<8><<<grid, block, 0, s>>>(a); break;
    default: calibrate_read_kernel<0><<<grid, block, 0, s>>>(a); break;
  }
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
