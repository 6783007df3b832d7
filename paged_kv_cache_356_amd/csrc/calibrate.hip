// calibrate.hip — the read-bandwidth reference: read the listed K/V tiles of two pools and nothing
// else (no products, no softmax, no stores beyond one word per wavefront), so that the decode
// kernels' achieved bandwidth can be set against a plain read of the same bytes on this device.
//
// Wavefront w of W reads list entries [w n / W, (w + 1) n / W), each tile in 1 KiB units (64
// lanes x 16 bytes), K then V, through two batches of 8 loads per lane: one batch is consumed
// while the other is in flight.
#include <hip/hip_runtime.h>

#include "pa_calibrate.h"

namespace {

constexpr int kBatch = 8;

struct CalArgs {
  const char *k_pool, *v_pool;
  int64_t tile_bytes;
  const int32_t *tiles;
  int64_t num_tiles;
  uint32_t *sink;
  int32_t num_waves;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Unit j (of n) of a round whose tile indices sit one per lane in `ids`: chunk j % c of pool
// (j / c) % 2 of the round's tile j / (2 c).  Past n: zeros, no load.
__device__ __forceinline__ u32x4_t load_unit(const CalArgs &a, int ids, int j, int n) {
  if (j >= n) return u32x4_t{0, 0, 0, 0};
  const int c = (int)(a.tile_bytes >> 10);
  const int e = j / (2 * c), r = j - e * 2 * c;
  const int64_t t = __builtin_amdgcn_readlane(ids, e);
  const char *pool = r < c ? a.k_pool : a.v_pool;
  const u32x4_t *p =
      reinterpret_cast<const u32x4_t *>(pool + t * a.tile_bytes + (int64_t)(r % c) * 1024) +
      (threadIdx.x & 63);
  return __builtin_nontemporal_load(p);
}

__global__ __launch_bounds__(256) void calibrate_read_kernel(CalArgs a) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.num_waves) return;
  const int lane = threadIdx.x & 63;
  const int64_t t0 = w * a.num_tiles / a.num_waves, t1 = (w + 1) * a.num_tiles / a.num_waves;
  const int c2 = (int)(a.tile_bytes >> 9);  // units per tile (K and V)
  uint32_t acc = 0;
  // Rounds of up to 64 tiles: their indices one per lane, then the round's units through two
  // batches of kBatch loads, one consumed while the other is in flight.
  for (int64_t tb = t0; tb < t1; tb += 64) {
    const int nk = (int)min((int64_t)64, t1 - tb);
    const int ids = lane < nk ? (a.tiles ? a.tiles[tb + lane] : (int)(tb + lane)) : 0;
    const int n = nk * c2;
    u32x4_t x[kBatch], y[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) x[i] = load_unit(a, ids, i, n);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) y[i] = load_unit(a, ids, kBatch + i, n);
    for (int j = 0; j < n; j += 2 * kBatch) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        acc ^= x[i].x ^ x[i].y ^ x[i].z ^ x[i].w;
        x[i] = load_unit(a, ids, j + 2 * kBatch + i, n);
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        acc ^= y[i].x ^ y[i].y ^ y[i].z ^ y[i].w;
        y[i] = load_unit(a, ids, j + 3 * kBatch + i, n);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane == 0) a.sink[w] = acc;
}

}  // namespace

extern "C" pa_status pa_calibrate_read(const void *k_pool, const void *v_pool, int64_t tile_bytes,
                                       const int32_t *tiles, int64_t num_tiles, uint32_t *sink,
                                       int32_t num_waves, void *stream) {
  if (!k_pool || !v_pool || !sink) return PA_ERR_NULL;
  if (tile_bytes <= 0 || tile_bytes % 1024 != 0 || num_tiles < 0 || num_waves < 1)
    return PA_ERR_SHAPE;
  if (num_tiles == 0) return PA_OK;
  CalArgs a;
  a.k_pool = static_cast<const char *>(k_pool);
  a.v_pool = static_cast<const char *>(v_pool);
  a.tile_bytes = tile_bytes;
  a.tiles = tiles;
  a.num_tiles = num_tiles;
  a.sink = sink;
  a.num_waves = num_waves;
  const unsigned grid = (unsigned)((num_waves + 3) / 4);
  calibrate_read_kernel<<<dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
