// partition_reduce.hip — merge the split-K partitions of paged decode attention.
//
// Partition p of a sequence produced, for each query head, its running max m_p (base-2 logits),
// its running sum l_p of 2^(z - m_p) and its normalised output o_p.  The whole-sequence result is
//   M = max_p m_p,  w_p = l_p * 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p,
// the same online-softmax merge the partitions used inside ("PagedAttention" (devoured.fyi), "Why
// the attention kernel works at all": attention walks K and V one chunk at a time).
// Sequences that fit one partition were finished by the decode kernel and are skipped here.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kMaxPartsInLds = 1024;

template <class QT>
__global__ __launch_bounds__(128) void partition_reduce_kernel(DecodeArgs a) {
  __shared__ float w_s[kMaxPartsInLds];
  __shared__ float red_s[2];
  const int hq = blockIdx.x, s = blockIdx.y;
  const int D = a.cache.head_dim;
  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int PT = a.partition_size;
  const int np = (Ls + PT - 1) / PT;
  if (np <= 1) return;
  const size_t row0 = ((size_t)s * a.num_q_heads + hq) * a.num_partitions;
  const float *ml = a.part_ml + row0 * 2;
  const int tid = threadIdx.x;

  // global max over partitions (np <= num_partitions; loops cover any count)
  float M = -INFINITY;
  for (int p = tid; p < np; p += blockDim.x) M = fmaxf(M, ml[2 * p]);
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((tid & 63) == 0) red_s[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(red_s[0], red_s[1]);

  float wsum = 0.0f;
  for (int p = tid; p < np; p += blockDim.x) {
    const float mp = ml[2 * p];
    const float wp = (mp == -INFINITY) ? 0.0f : ml[2 * p + 1] * __builtin_amdgcn_exp2f(mp - M);
    if (p < kMaxPartsInLds) w_s[p] = wp;
    wsum += wp;
  }
  for (int o = 32; o >= 1; o >>= 1) wsum += __shfl_xor(wsum, o);
  __syncthreads();
  if ((tid & 63) == 0) red_s[tid >> 6] = wsum;
  __syncthreads();
  wsum = red_s[0] + red_s[1];
  const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;

  auto *out = static_cast<typename QT::raw *>(a.out) + ((size_t)s * a.num_q_heads + hq) * D;
  const float *po = a.part_out + row0 * D;
  for (int d = tid; d < D; d += blockDim.x) {
    float acc = 0.0f;
    for (int p = 0; p < np; ++p) {
      float wp;
      if (p < kMaxPartsInLds) {
        wp = w_s[p];
      } else {
        const float mp = ml[2 * p];
        wp = (mp == -INFINITY) ? 0.0f : ml[2 * p + 1] * __builtin_amdgcn_exp2f(mp - M);
      }
      acc += wp * po[(size_t)p * D + d];
    }
    out[d] = from_f32<QT>(acc * inv);
  }
}

}  // namespace

hipError_t launch_partition_reduce(const DecodeArgs &a, hipStream_t s) {
  if (a.num_partitions <= 1) return hipSuccess;
  dim3 grid(a.num_q_heads, a.num_seqs), block(128);
  switch (a.q_dtype) {
    case kF32: partition_reduce_kernel<f32_t><<<grid, block, 0, s>>>(a); break;
    case kF16: partition_reduce_kernel<f16_t><<<grid, block, 0, s>>>(a); break;
    case kBF16: partition_reduce_kernel<bf16_t><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
