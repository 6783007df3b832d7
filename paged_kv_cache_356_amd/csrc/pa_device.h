// pa_device.h — device-side helpers shared by the gfx950 kernels of libpa.so: element types,
// exact conversions, the E4M3FN fp8 codec and the pool-layout address arithmetic described in
// include/pa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kernels.h"

namespace pa {

// Cache element tags.  bf16 and fp8 are carried as raw bits; conversions below are exact.
struct f32_t { using raw = float; static constexpr int bytes = 4; };
struct f16_t { using raw = _Float16; static constexpr int bytes = 2; };
struct bf16_t { using raw = uint16_t; static constexpr int bytes = 2; };
struct fp8_t { using raw = uint8_t; static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// binary32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E4M3FN byte -> binary32 (exact).  S.1111.111 is NaN; no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t ex = (c >> 3) & 0xfu, fr = c & 0x7u;
  float v;
  if (ex == 0) {
    v = (float)fr * 0.001953125f;  // fr * 2^-9 (exact)
  } else {
    v = __uint_as_float(((ex + 120u) << 23) | (fr << 20));
  }
  if (ex == 15u && fr == 7u) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | sign);
}

// binary32 -> E4M3FN byte: round to nearest, ties to even; |x| >= 448 saturates to 448; NaN -> 0x7F
// with the input's sign.  Integer arithmetic only, so the result does not depend on the FPU mode.
__device__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu);
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);  // 448.0f and above
  uint32_t code;
  if (a < 0x3c800000u) {  // below 2^-6: subnormal codes, steps of 2^-9
    // a * 2^9 is exact (power-of-two scaling of a value < 2^-6); round half to even.
    const float q = __uint_as_float(a) * 512.0f;
    code = (uint32_t)__builtin_rintf(q);  // 0 .. 8; 8 is the smallest normal code 0x08
  } else {
    // keep 3 fraction bits of 23, round half to even, then rebias 127 -> 7
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    r &= ~0xfffffu;
    const uint32_t ex = (r >> 23) - 120u;
    code = (ex << 3) | ((r >> 20) & 7u);
  }
  return (uint8_t)(sign | code);
}

template <class T> __device__ __forceinline__ float load_f32(const typename T::raw *p, size_t i);
template <> __device__ __forceinline__ float load_f32<f32_t>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f32<f16_t>(const _Float16 *p, size_t i) {
  return (float)p[i];
}
template <> __device__ __forceinline__ float load_f32<bf16_t>(const uint16_t *p, size_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <class T> __device__ __forceinline__ typename T::raw from_f32(float x);
template <> __device__ __forceinline__ float from_f32<f32_t>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<f16_t>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ uint16_t from_f32<bf16_t>(float x) {
  return f32_to_bf16_bits(x);
}

// Raw-element -> float for cache elements (fp8 without its scale).
template <class T> __device__ __forceinline__ float cache_to_f32(typename T::raw v);
template <> __device__ __forceinline__ float cache_to_f32<f32_t>(float v) { return v; }
template <> __device__ __forceinline__ float cache_to_f32<f16_t>(_Float16 v) { return (float)v; }
template <> __device__ __forceinline__ float cache_to_f32<bf16_t>(uint16_t v) {
  return bf16_bits_to_f32(v);
}
template <> __device__ __forceinline__ float cache_to_f32<fp8_t>(uint8_t v) { return e4m3_to_f32(v); }

// Pool layout (include/pa.h), B positions per block.  E = 16 / bytes elements per 16-byte vector.
// K tile: element (t, i) at ((i / E) * B + t) * E + i % E;  V tile: element (t, i) at i * B + t.
template <int BYTES>
struct Layout {
  static constexpr int E = 16 / BYTES;
  __device__ __forceinline__ static size_t tile(int64_t block, int h, int H, int D, int B) {
    return ((size_t)block * H + h) * (size_t)B * D;
  }
  __device__ __forceinline__ static int k_off(int t, int i, int B) {
    return ((i / E) * B + t) * E + (i % E);
  }
  __device__ __forceinline__ static int v_off(int t, int i, int B) { return i * B + t; }
};

}  // namespace pa
