// mfma_common.h — device pieces shared by the matrix-core decode (decode_mfma.hip) and the paged
// prefill (prefill_mfma.hip): tile descriptors, the MFMA products and their operand types, the
// fp8 widening, a wavefront's row state and query operand, the output of finished rows, and the
// LDS stages with their barrier.
//
// The thread and workgroup indices come straight from the compiler builtins rather than from HIP's
// index objects, whose device-library helpers are not inlined into code compiled with other
// floating-point options than the library's (the prefill's translation unit is).
#pragma once

#include <type_traits>
#include <utility>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int block_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
// workgroups in the launch: the dispatch packet's grid size over the 256-thread workgroups every
// kernel of the library uses
__device__ __forceinline__ int grid_x() {
  using cu32 = const __attribute__((address_space(4))) uint32_t;
  return (int)(((cu32 *)__builtin_amdgcn_dispatch_ptr())[3] / 256u);
}

constexpr int kWaves = 4;

#define PA_LDS __attribute__((address_space(3)))  // LDS pointers

// K/V tiles are read with raw buffer loads through a descriptor per tile: a slot with no block
// gets a descriptor of length 0, whose loads return zeros without touching memory (and still count
// in vmcnt, so the waits on the loads behind them stay partial).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;  // 32-bit data format, the value raw loads use on gfx9

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *tile, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(tile), (short)0, bytes, kRsrcWord3);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNoMax = -3.0e38f;  // running-maximum floor (finite)
constexpr float kSlack = 8.0f;  // base-2 headroom of the lazily rescaled running maximum

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ f4_t mma_k32(uint4 a, uint4 b, f4_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f4_t mma_k16(uint2 a, uint2 b, f4_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a),
                                                     __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a),
                                                 __builtin_bit_cast(h4_t, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values of the MFMA input type (round to nearest even), packed.
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  if constexpr (BF) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)y) << 16);
  } else {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)y) << 16);
  }
}

// The same rounding in one packed conversion (v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
template <bool BF>
__device__ __forceinline__ uint32_t pack2_pk(float x, float y) {
  typedef float fl2_t __attribute__((ext_vector_type(2)));
  if constexpr (BF) {
    typedef __bf16 bh2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2_t){x, y}, bh2_t));
  } else {
    typedef _Float16 hh2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2_t){x, y}, hh2_t));
  }
}

template <bool BF>
__device__ __forceinline__ float unpack_lo(uint32_t v) {
  if constexpr (BF) return __uint_as_float(v << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
template <bool BF>
__device__ __forceinline__ float unpack_hi(uint32_t v) {
  if constexpr (BF) return __uint_as_float(v & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

// Four E4M3FN bytes (byte 0 first) -> four binary16 values equal to decode(byte), by the hardware
// conversion v_cvt_scalef32_pk_f16_fp8 at scale 1 (exact for all 256 codes, checked on the GPU;
// the NaN code gives a NaN).
__device__ __forceinline__ uint2 e4m3x4_to_f16x4(uint32_t x) {
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
  return r;
}

template <class CT, int D>
struct Frag {
  static constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  static constexpr int kKLoads = kFP8 ? D / 64 : D / 32;  // 16-byte K loads per lane
  static constexpr int kNT = D / 16;                      // PV products (16 head-dim rows each)
  using VRaw = typename std::conditional<kFP8, uint32_t, uint2>::type;
  uint4 k[kKLoads];
  VRaw v[kNT];
};


// ---------------------------------------------------------------------------------------------
// Per-wavefront pieces.  Lane l = 16 * grp + col: column col of the products is one query row.

template <int D>
struct RowState {
  uint4 qop[D / 32];  // Q^T operand of this lane's query row
  float m, l;         // running maximum (base-2 logits) and running sum of this lane's column
  f4_t acc[D / 16];   // O^T accumulator: head-dim rows 16 nt + 4 grp + i of this lane's column
};

// Q^T operand: lane l holds query row (rs, rhq), 8 dims per product kk, zeros for a padding
// column.  The dims follow the K operand: f16/bf16 tiles give lane group grp dims 8 grp + 32 kk;
// fp8 tiles give 16-byte vectors of 16 dims, split in two products, so 16 grp + 64 (kk/2) +
// 8 (kk%2).
template <class CT, int D>
__device__ __forceinline__ void load_query(const DecodeArgs &a, int rs, int rhq, bool rvalid,
                                           RowState<D> &st) {
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  const int grp = (thread_x() & 63) >> 4;
  const auto *q =
      reinterpret_cast<const uint16_t *>(a.q) + (size_t)rs * a.q_stride + (size_t)rhq * D;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const int d0 = kFP8 ? 16 * grp + 64 * (kk >> 1) + 8 * (kk & 1) : 8 * grp + 32 * kk;
    st.qop[kk] = rvalid ? *reinterpret_cast<const uint4 *>(q + d0) : make_uint4(0, 0, 0, 0);
  }
  st.m = kNoMax;  // a finite floor: a fully masked block gives exp2(-inf - m) = 0, not NaN
  st.l = 0.0f;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) st.acc[nt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// Lane i's entry of the first 64 blocks [jb0, jb1) of a table row (-1 past the range).
__device__ __forceinline__ int first_table_entries(const int32_t *table, int jb0, int jb1) {
  const int lane = thread_x() & 63;
  return lane < min(64, jb1 - jb0) ? table[jb0 + lane] : -1;
}

// The per-head scales are read through the constant address space: the kernel never writes them,
// and scalar loads keep them out of the vector memory counter the block ring waits on.
template <class CT>
__device__ __forceinline__ void head_scales(const DecodeArgs &a, int h, float &kscale,
                                            float &vscale) {
  kscale = a.scale * kLog2e;
  vscale = 1.0f;
  if constexpr (std::is_same<CT, fp8_t>::value) {
    using cfloat = const __attribute__((address_space(4))) float;
    kscale *= ((cfloat *)(uintptr_t)a.cache.k_scale)[h];
    vscale = ((cfloat *)(uintptr_t)a.cache.v_scale)[h];
  }
}

__device__ __forceinline__ int clamp_len(const DecodeArgs &a, int s) {
  int L = a.context_lens[s];
  return L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
}

// A 4-, 8- or 16-byte LDS read.
template <class T>
__device__ __forceinline__ T lds_load(const PA_LDS char *p) {
  if constexpr (sizeof(T) == 16) return __builtin_bit_cast(T, *(const PA_LDS u32x4_t *)p);
  else if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, *(const PA_LDS u32x2_t *)p);
  else return __builtin_bit_cast(T, *(const PA_LDS uint32_t *)p);
}

// A finished row state to the output (slot < 0, scaled by vscale) or to workspace partition
// `slot` (scaled by pvscale).
template <class QT, int D>
__device__ __forceinline__ void emit_rows(const DecodeArgs &a, const RowState<D> &st, float vscale,
                                          float pvscale, int slot, int rs, int rhq, bool rvalid) {
  constexpr int NT = D / 16;
  const int Hq = a.num_q_heads;
  const int grp = (thread_x() & 63) >> 4;
  // the row's sum over the four lane groups; m is already uniform over them
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!rvalid) return;
  const size_t orow = (size_t)rs * Hq + rhq;
  const float inv = l > 0.0f ? (slot < 0 ? vscale : pvscale) / l : 0.0f;  // no position: zero
  if (slot < 0) {
    auto *out = static_cast<typename QT::raw *>(a.out) + orow * D;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      typename QT::raw v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<QT>(st.acc[nt][i] * inv);
      *reinterpret_cast<uint2 *>(out + 16 * nt + 4 * grp) = *reinterpret_cast<const uint2 *>(v);
    }
  } else {
    const size_t row = orow * a.num_partitions + slot;
    if constexpr (std::is_same<QT, f16_t>::value) {
      // f16 queries: the partial output in fp16 (half the workspace traffic; it is a normalised
      // average of V rows, rounded once more before the merge), stored lane-contiguous: the
      // quads of head dims 16 nt + 4 grp .. + 3 at quad grp * NT + nt of the row, so each lane
      // writes NT * 8 contiguous bytes and a row's four lane groups one contiguous span
      typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
      uint32_t hw[2 * NT];  // round to nearest even
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        hw[2 * nt] = __builtin_bit_cast(
            uint32_t, h2_t{(_Float16)(st.acc[nt][0] * inv), (_Float16)(st.acc[nt][1] * inv)});
        hw[2 * nt + 1] = __builtin_bit_cast(
            uint32_t, h2_t{(_Float16)(st.acc[nt][2] * inv), (_Float16)(st.acc[nt][3] * inv)});
      }
      uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<_Float16 *>(a.part_out) + row * D +
                                             (size_t)grp * NT * 4);
#pragma unroll
      for (int k = 0; k < NT / 2; ++k)
        dst[k] = make_uint4(hw[4 * k], hw[4 * k + 1], hw[4 * k + 2], hw[4 * k + 3]);
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float4 v;
        v.x = st.acc[nt][0] * inv;
        v.y = st.acc[nt][1] * inv;
        v.z = st.acc[nt][2] * inv;
        v.w = st.acc[nt][3] * inv;
        *reinterpret_cast<float4 *>(a.part_out + row * D + 16 * nt + 4 * grp) = v;
      }
    }
    if (grp == 0) {
      a.part_ml[row * 2] = st.m;
      a.part_ml[row * 2 + 1] = l;
    }
  }
}

// f(std::integral_constant<int, i>) for i = I .. N - 1, in order.
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int kBytes, int I>
__device__ __forceinline__ PA_LDS char *prefix_stage() {
  __shared__ __attribute__((aligned(16))) char stage[kBytes];
  return (PA_LDS char *)stage;
}

// Wait until at most N of this wavefront's memory reads are outstanding (its LDS copies land in
// order), then for its LDS reads, then meet the workgroup.  The memory clobber keeps the compiler
// from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
}  // namespace
}  // namespace pa
