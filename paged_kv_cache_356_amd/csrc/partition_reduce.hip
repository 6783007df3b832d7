// partition_reduce.hip — merge the split-K partitions of paged decode attention.
//
// Partition p of a sequence produced, for each query head, its running max m_p (base-2 logits),
// its running sum l_p of 2^(z - m_p) and its normalised output o_p.  The whole-sequence result is
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p,
// the same online-softmax merge the partitions used inside ("PagedAttention" (devoured.fyi), "Why
// the attention kernel works at all": attention walks K and V one chunk at a time).
// Sequences that fit one partition of the plain decode were finished by the decode kernel and are
// skipped here; with a shared prefix every row is merged (its prefix chunks and its suffix
// partitions).
//
// One wavefront per (sequence, query head) row, four rows per workgroup, no barriers.  Each lane
// owns one float4 column of the partial outputs (C = D / 4 columns) and the partitions
// lane / C, lane / C + G, ... (G = 64 / C) of a chunk of 64; the weights of the chunk's partitions
// sit one per lane and are fetched with lane shuffles, the loads of a sub-chunk of kPer * G
// partitions are all issued before any is used, and the G column groups are combined with shuffles
// at the end.
// The first chunk's (m, l) pairs and first sub-chunk of outputs are loaded together, as soon as the
// row's partition count is known: the outputs do not wait for the maximum, so a row with few
// partitions makes two round trips to memory (context length, then its partials), not three.
// Slots past the row's partitions hold whatever earlier calls left there and are never read.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kRowsPerGroup = 4;

// Head dims 4 c .. 4 c + 3 of partial output p of a row (its first quad at q0), fp32 or fp16
// (kHalf).  fp16 partials are stored lane-contiguous by the decode kernel: the quad of dims
// 16 nt + 4 grp .. sits at quad grp * (D / 16) + nt.
template <bool kHalf, int D>
__device__ __forceinline__ float4 load_part4(const float *part_out, size_t q0, int p, int c) {
  constexpr int C = D / 4;
  if constexpr (kHalf) {
    const int q = (c & 3) * (D / 16) + (c >> 2);
    const uint2 u = reinterpret_cast<const uint2 *>(part_out)[q0 + (size_t)p * C + q];
    const _Float16 *h = reinterpret_cast<const _Float16 *>(&u);
    return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
  } else {
    return reinterpret_cast<const float4 *>(part_out)[q0 + (size_t)p * C + c];
  }
}
// Split variant: wavefronts per row, and the most rows it is used for.
constexpr int kWavesSplit = 4;
constexpr int kSplitRows = 1024;

// kPer: float4 loads in flight per lane (a sub-chunk of G * kPer partitions).  A few keep the
// registers low, so that many rows are in flight, for batches of many rows (4: 8 and 16 measured
// no better); 32 takes 64 partitions of a row in one round trip when rows are few (the wide
// variant: then occupancy does not matter).
constexpr int kPerNarrow = 4;
// Scale of the merged row: 1, or the KV head's v_scale where the partials are in units of fp8
// cache codes (part_vscale).
template <bool kHalf>
__device__ __forceinline__ float out_scale(const DecodeArgs &a, int row) {
  if constexpr (kHalf)
    if (a.part_vscale) {
      const int hq = row % a.num_q_heads;
      return a.cache.v_scale[hq / (a.num_q_heads / a.cache.num_kv_heads)];
    }
  return 1.0f;
}

// Output row (s * Hq + hq) of grid row r: with a dealing order, grid rows run over the sequences
// in that order (the decode's largest items first, so that the rows with the most partitions are
// merged first), else in batch order; -1 for an order entry outside the batch.  The entry is the
// same for the whole wavefront, so the order is read with a scalar load.
__device__ __forceinline__ int reduce_row(const DecodeArgs &a, int r) {
  if (!a.seq_order) return r;
  const int Hq = a.num_q_heads;
  const int e = __builtin_amdgcn_readfirstlane(r / Hq);
  const int s = a.seq_order[e];
  return (unsigned)s < (unsigned)a.num_seqs ? s * Hq + (r - e * Hq) : -1;
}

template <class QT, int D, int kPer, bool kHalf>
__global__ __launch_bounds__(64 * kRowsPerGroup) void partition_reduce_kernel(DecodeArgs a) {
  constexpr int C = D / 4;   // float4 columns of a partial output
  constexpr int G = 64 / C;  // partitions handled side by side in a wavefront
  constexpr int SUB = G * kPer;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
  if (r >= a.num_seqs * a.num_q_heads) return;
  const int row = reduce_row(a, r);  // s * Hq + hq
  if (row < 0) return;
  const int s = row / a.num_q_heads;
  const int NP = a.num_partitions;
  const size_t row0 = (size_t)row * NP;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml) + row0;
  const size_t po0 = row0 * C;  // float4 index of the row's first partial
  const int c = lane % C, grp = lane / C;

  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int np = row_partitions(a, Ls);
  if (np <= 1 && a.prefix_len == 0) return;  // finished by the decode kernel
  const float2 v0 = lane < np ? ml[lane] : make_float2(-INFINITY, 0.0f);
  float4 x[kPer];  // one sub-chunk of partial outputs; the first is loaded beside v0
  auto load_sub = [&](int base, int sub, int n) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = sub + grp + k * G;
      x[k] = q < n ? load_part4<kHalf, D>(a.part_out, po0, base + q, c)
                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  load_sub(0, 0, min(64, np));

  // M = max over the row's partitions
  float M = v0.x;
  for (int p = lane + 64; p < np; p += 64) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float wsum = 0.0f;
  for (int base = 0; base < np; base += 64) {
    const int n = min(64, np - base);
    const float2 v = base == 0 ? v0 : (lane < n ? ml[base + lane] : make_float2(-INFINITY, 0.0f));
    const float wl = v.x == -INFINITY ? 0.0f : v.y * __builtin_amdgcn_exp2f(v.x - M);
    wsum += wl;
    for (int sub = 0; sub < n; sub += SUB) {
      if (base > 0 || sub > 0) load_sub(base, sub, n);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float wq = __shfl(wl, (sub + grp + k * G) & 63);  // 0 for q >= n
        acc.x += wq * x[k].x;
        acc.y += wq * x[k].y;
        acc.z += wq * x[k].z;
        acc.w += wq * x[k].w;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
#pragma unroll
  for (int o = C; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
  }
  if (lane < C) {
    const float inv = wsum > 0.0f ? out_scale<kHalf>(a, row) / wsum : 0.0f;
    auto *out = static_cast<typename QT::raw *>(a.out) + (size_t)row * D + 4 * lane;
    out[0] = from_f32<QT>(acc.x * inv);
    out[1] = from_f32<QT>(acc.y * inv);
    out[2] = from_f32<QT>(acc.z * inv);
    out[3] = from_f32<QT>(acc.w * inv);
  }
}

// Few rows with many partitions: one workgroup per row, its four wavefronts each merging a quarter
// of the head dims, so that the same bytes are read by four times as many wavefronts.  In a
// wavefront, lane (group pg, column c) owns float4 column c of the quarter and the partitions
// pg, pg + 8, ... (up to 8 of them per pass, all loaded before any is used); the eight groups are
// combined with shuffles at the end.
template <class QT, int D, bool kHalf>
__global__ __launch_bounds__(256) void partition_reduce_split_kernel(DecodeArgs a) {
  constexpr int C = D / 4 / kWavesSplit;  // float4 columns per wavefront
  constexpr int PG = 64 / C;              // partition groups per wavefront
  constexpr int kPer = 64 / PG;           // partitions per lane in one pass of 64
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = reduce_row(a, blockIdx.x);  // s * Hq + hq
  if (row < 0) return;
  const int s = row / a.num_q_heads;
  const int NP = a.num_partitions;
  const size_t row0 = (size_t)row * NP;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml) + row0;
  const size_t po0 = row0 * (D / 4);  // float4 index of the row's first partial
  const int c = lane % C, pg = lane / C;
  const int col = w * C + c;  // float4 column of the row

  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int np = row_partitions(a, Ls);
  if (np <= 1 && a.prefix_len == 0) return;  // finished by the decode kernel
  const float2 v0 = lane < np ? ml[lane] : make_float2(-INFINITY, 0.0f);
  float4 x[kPer];
  auto load_pass = [&](int base, int n) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = pg + k * PG;
      x[k] = q < n ? load_part4<kHalf, D>(a.part_out, po0, base + q, col)
                   : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
  };
  load_pass(0, min(64, np));
  float M = v0.x;
  for (int p = lane + 64; p < np; p += 64) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float wsum = 0.0f;
  for (int base = 0; base < np; base += 64) {
    const int n = min(64, np - base);
    if (base > 0) load_pass(base, n);
    const float2 v = base == 0 ? v0 : (lane < n ? ml[base + lane] : make_float2(-INFINITY, 0.0f));
    const float wl = v.x == -INFINITY ? 0.0f : v.y * __builtin_amdgcn_exp2f(v.x - M);
    wsum += wl;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float wq = __shfl(wl, (pg + k * PG) & 63);  // 0 for q >= n
      acc.x += wq * x[k].x;
      acc.y += wq * x[k].y;
      acc.z += wq * x[k].z;
      acc.w += wq * x[k].w;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
#pragma unroll
  for (int o = C; o < 64; o <<= 1) {
    acc.x += __shfl_xor(acc.x, o);
    acc.y += __shfl_xor(acc.y, o);
    acc.z += __shfl_xor(acc.z, o);
    acc.w += __shfl_xor(acc.w, o);
  }
  if (pg == 0) {
    const float inv = wsum > 0.0f ? out_scale<kHalf>(a, row) / wsum : 0.0f;
    auto *out = static_cast<typename QT::raw *>(a.out) + (size_t)row * D + 4 * col;
    out[0] = from_f32<QT>(acc.x * inv);
    out[1] = from_f32<QT>(acc.y * inv);
    out[2] = from_f32<QT>(acc.z * inv);
    out[3] = from_f32<QT>(acc.w * inv);
  }
}

template <class QT, bool kHalf>
hipError_t launch_qh(const DecodeArgs &a, hipStream_t s) {
  const int rows = a.num_seqs * a.num_q_heads;
  dim3 grid((rows + kRowsPerGroup - 1) / kRowsPerGroup), block(64 * kRowsPerGroup);
  const bool wide = rows <= 2048 && a.num_partitions > 16;
  if (wide && rows <= kSplitRows) {
    if (a.cache.head_dim == 64)
      partition_reduce_split_kernel<QT, 64, kHalf><<<dim3(rows), dim3(64 * kWavesSplit), 0, s>>>(a);
    else
      partition_reduce_split_kernel<QT, 128, kHalf><<<dim3(rows), dim3(64 * kWavesSplit), 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.cache.head_dim == 64) {
    if (wide) partition_reduce_kernel<QT, 64, 16, kHalf><<<grid, block, 0, s>>>(a);
    else partition_reduce_kernel<QT, 64, 2, kHalf><<<grid, block, 0, s>>>(a);
  } else {
    if (wide) partition_reduce_kernel<QT, 128, 32, kHalf><<<grid, block, 0, s>>>(a);
    else partition_reduce_kernel<QT, 128, kPerNarrow, kHalf><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

// fp16 partials come only from the matrix-core kernel with f16 queries (part_f16).
template <class QT>
hipError_t launch_q(const DecodeArgs &a, hipStream_t s) {
  if constexpr (std::is_same<QT, f16_t>::value)
    if (a.part_f16) return launch_qh<QT, true>(a, s);
  return launch_qh<QT, false>(a, s);
}

}  // namespace

hipError_t launch_partition_reduce(const DecodeArgs &a, hipStream_t s) {
  if (a.num_partitions <= 1 && a.prefix_len == 0) return hipSuccess;
  switch (a.q_dtype) {
    case kF32: return launch_q<f32_t>(a, s);
    case kF16: return launch_q<f16_t>(a, s);
    case kBF16: return launch_q<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
