// partition_reduce.hip — merge the split-K partitions of paged decode attention.
//
// Partition p of a sequence produced, for each query head, its running max m_p (base-2 logits),
// its running sum l_p of 2^(z - m_p) and its normalised output o_p.  The whole-sequence result is
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p,
// the same online-softmax merge the partitions used inside ("PagedAttention" (devoured.fyi), "Why
// the attention kernel works at all": attention walks K and V one chunk at a time).
// Sequences that fit one partition were finished by the decode kernel and are skipped here.
//
// One workgroup of 256 threads per (sequence, query head) row.  The row's partials are read as
// float4 columns: thread t owns column t % C (C = D / 4) and partitions t / C, t / C + G, ...
// (G = 256 / C), so every load of a chunk of 256 partitions is issued before any is used; the G
// per-thread sums are then combined through LDS.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;  // partitions whose weights are staged in LDS at a time

template <class QT, int D>
__global__ __launch_bounds__(kThreads) void partition_reduce_kernel(DecodeArgs a) {
  constexpr int C = D / 4;            // float4 columns of a partial output
  constexpr int G = kThreads / C;     // partitions handled side by side
  constexpr int kPer = kChunk / G;    // partitions per thread and chunk
  __shared__ float w_s[kChunk];
  __shared__ float red_s[kThreads / 64];
  __shared__ float4 acc_s[G][C];

  const int row = blockIdx.x;  // s * Hq + hq
  const int s = row / a.num_q_heads;
  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int PT = a.partition_size;
  const int np = (Ls + PT - 1) / PT;
  if (np <= 1) return;
  const size_t row0 = (size_t)row * a.num_partitions;
  const float2 *ml = reinterpret_cast<const float2 *>(a.part_ml) + row0;
  const float4 *po = reinterpret_cast<const float4 *>(a.part_out) + row0 * C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // M = max over partitions
  float M = -INFINITY;
  for (int p = tid; p < np; p += kThreads) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red_s[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));

  const int c = tid % C, grp = tid / C;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float wsum = 0.0f;
  for (int base = 0; base < np; base += kChunk) {
    const int n = min(kChunk, np - base);
    __syncthreads();  // previous chunk's weights are no longer read
    if (tid < n) {
      const float2 v = ml[base + tid];
      const float wp = v.x == -INFINITY ? 0.0f : v.y * __builtin_amdgcn_exp2f(v.x - M);
      w_s[tid] = wp;
      wsum += wp;
    }
    __syncthreads();
    float4 x[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int p = grp + k * G;
      x[k] = p < n ? po[(size_t)(base + p) * C + c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int p = grp + k * G;
      const float wp = p < n ? w_s[p] : 0.0f;
      acc.x += wp * x[k].x;
      acc.y += wp * x[k].y;
      acc.z += wp * x[k].z;
      acc.w += wp * x[k].w;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
  __syncthreads();
  if (lane == 0) red_s[wv] = wsum;
  acc_s[grp][c] = acc;
  __syncthreads();
  if (tid < C) {
    const float tot = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
    const float inv = tot > 0.0f ? 1.0f / tot : 0.0f;
    float4 r = acc_s[0][tid];
#pragma unroll
    for (int k = 1; k < G; ++k) {
      r.x += acc_s[k][tid].x;
      r.y += acc_s[k][tid].y;
      r.z += acc_s[k][tid].z;
      r.w += acc_s[k][tid].w;
    }
    auto *out = static_cast<typename QT::raw *>(a.out) + (size_t)row * D + 4 * tid;
    out[0] = from_f32<QT>(r.x * inv);
    out[1] = from_f32<QT>(r.y * inv);
    out[2] = from_f32<QT>(r.z * inv);
    out[3] = from_f32<QT>(r.w * inv);
  }
}

template <class QT>
hipError_t launch_q(const DecodeArgs &a, hipStream_t s) {
  dim3 grid(a.num_seqs * a.num_q_heads), block(kThreads);
  if (a.cache.head_dim == 64) partition_reduce_kernel<QT, 64><<<grid, block, 0, s>>>(a);
  else partition_reduce_kernel<QT, 128><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partition_reduce(const DecodeArgs &a, hipStream_t s) {
  if (a.num_partitions <= 1) return hipSuccess;
  switch (a.q_dtype) {
    case kF32: return launch_q<f32_t>(a, s);
    case kF16: return launch_q<f16_t>(a, s);
    case kBF16: return launch_q<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
