// decode_valu.hip — split-K paged decode attention on the vector ALUs (all cache dtypes).
//
// The kernel walks each sequence's block table and gathers one 16-token block of K and V at a time
// ("PagedAttention" (devoured.fyi), "PagedAttention in one picture" and "Why the attention kernel
// works at all"); it computes ordinary softmax(q K^T * scale) V ("Misconceptions": the math is
// unchanged).  Long contexts are cut into partitions of `partition_size` tokens; each workgroup
// produces one partition's (running max, running sum, normalised output) with an online softmax,
// and pa_partition_reduce merges them.
//
// Workgroup = 4 wavefronts for one (partition, KV head, sequence); the wavefronts take the
// partition's blocks round-robin, each with its own online-softmax state, and are merged in LDS.
// Inside a wavefront, QK^T uses lane = 4 * token + quarter (each lane dots one quarter of the head
// dimension for all grouped query heads, then a 4-lane reduction); PV uses lane = head-dim index
// (each lane owns D / 64 output columns for every grouped query head).  Exponentials are base 2.
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;

template <class CT, class QT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
  using L = Layout<CT::bytes>;
  constexpr int E = L::E;
  constexpr int DQ = D / 4;        // head-dim slice per lane in QK^T
  constexpr int NPV = D / 64;      // output columns per lane in PV
  __shared__ float q_s[GMAX][D];
  __shared__ float p_s[kWaves][GMAX][kBlock];
  __shared__ float m_s[kWaves][GMAX], l_s[kWaves][GMAX];
  __shared__ float acc_s[kWaves][GMAX][D];

  const int s = blockIdx.z, h = blockIdx.y, part = blockIdx.x;
  const int H = a.cache.num_kv_heads, Hq = a.num_q_heads, g = Hq / H;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int PT = a.partition_size;
  const int nparts = (Ls + PT - 1) / PT;
  auto *out = static_cast<typename QT::raw *>(a.out);
  if (part >= nparts) {
    if (part == 0) {  // empty context: output is zero
      for (int x = tid; x < g * D; x += blockDim.x)
        out[((size_t)s * Hq + h * g) * D + x] = from_f32<QT>(0.0f);
    }
    return;
  }
  int start, end;
  partition_range(0, Ls, PT, part, &start, &end);

  const auto *q = static_cast<const typename QT::raw *>(a.q) + (size_t)s * a.q_stride +
                  (size_t)h * g * D;
  for (int x = tid; x < GMAX * D; x += blockDim.x) {
    const int i = x / D;
    q_s[i][x % D] = i < g ? load_f32<QT>(q, x) : 0.0f;
  }
  __syncthreads();

  float kscale = a.scale * kLog2e, vscale = 1.0f;
  if constexpr (std::is_same<CT, fp8_t>::value) {
    kscale *= a.cache.k_scale[h];
    vscale = a.cache.v_scale[h];
  }
  const auto *kpool = static_cast<const typename CT::raw *>(a.cache.k_pool);
  const auto *vpool = static_cast<const typename CT::raw *>(a.cache.v_pool);
  const int32_t *table = a.block_tables + (size_t)s * a.max_blocks_per_seq;

  const int t_qk = lane >> 2, quarter = lane & 3;
  float m[GMAX], l_loc[GMAX], acc[GMAX][NPV];
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    m[i] = -INFINITY;
    l_loc[i] = 0.0f;
#pragma unroll
    for (int k = 0; k < NPV; ++k) acc[i][k] = 0.0f;
  }

  const int jb0 = start / kBlock, jb1 = (end + kBlock - 1) / kBlock;
  for (int j = jb0 + w; j < jb1; j += kWaves) {
    const int bid = table[j];
    if ((unsigned)bid >= (unsigned)a.cache.num_blocks) continue;  // never dereferenced
    const size_t tile = L::tile(bid, h, H, D, kBlock);  // this kernel runs on 16-position blocks
    const int tok0 = j * kBlock;

    // ---- z[i] = scale * log2(e) * <q_i, k_t> for this lane's token t
    float part_dot[GMAX];
#pragma unroll
    for (int i = 0; i < GMAX; ++i) part_dot[i] = 0.0f;
#pragma unroll
    for (int cv = 0; cv < DQ / E; ++cv) {
      const int c = quarter * (DQ / E) + cv;  // 16-byte vector index along the head dimension
      union {
        uint4 v;
        typename CT::raw e[E];
      } kv;
      kv.v = *reinterpret_cast<const uint4 *>(kpool + tile + (size_t)(c * kBlock + t_qk) * E);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float kf = cache_to_f32<CT>(kv.e[e]);
#pragma unroll
        for (int i = 0; i < GMAX; ++i) part_dot[i] += q_s[i][c * E + e] * kf;
      }
    }
    const bool tok_ok = tok0 + t_qk < end;
    float z[GMAX], bmax[GMAX];
#pragma unroll
    for (int i = 0; i < GMAX; ++i) {
      float d = part_dot[i];
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      z[i] = tok_ok ? d * kscale : -INFINITY;  // select: NaN in tail slots never leaks
      float mx = z[i];
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      bmax[i] = mx;
    }
    // ---- online softmax update (all lanes hold the same m, alpha)
    float alpha[GMAX];
#pragma unroll
    for (int i = 0; i < GMAX; ++i) {
      const float mn = fmaxf(m[i], bmax[i]);
      alpha[i] = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m[i] - mn);
      const float p = mn == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(z[i] - mn);
      m[i] = mn;
      l_loc[i] = l_loc[i] * alpha[i] + (quarter == 0 ? p : 0.0f);
      if (quarter == 0) p_s[w][i][t_qk] = p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- acc[i][d] = alpha_i * acc[i][d] + sum_t p[i][t] * V[t][d]
#pragma unroll
    for (int k = 0; k < NPV; ++k) {
      const int d = lane + 64 * k;
      union {
        uint4 v[kBlock * CT::bytes / 16];
        typename CT::raw e[kBlock];
      } vv;
#pragma unroll
      for (int x = 0; x < kBlock * CT::bytes / 16; ++x)
        vv.v[x] = *reinterpret_cast<const uint4 *>(vpool + tile + (size_t)d * kBlock + x * (16 / CT::bytes));
      float vf[kBlock];
#pragma unroll
      for (int t = 0; t < kBlock; ++t) vf[t] = tok0 + t < end ? cache_to_f32<CT>(vv.e[t]) : 0.0f;
#pragma unroll
      for (int i = 0; i < GMAX; ++i) {
        float r = acc[i][k] * alpha[i];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) r += p_s[w][i][t] * vf[t];
        acc[i][k] = r;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the wavefronts: running sums are lane-partial, reduce them first
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    float x = l_loc[i];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (lane == 0) {
      m_s[w][i] = m[i];
      l_s[w][i] = x;
    }
#pragma unroll
    for (int k = 0; k < NPV; ++k) acc_s[w][i][lane + 64 * k] = acc[i][k];
  }
  __syncthreads();

  const int hq0 = h * g;
  for (int x = tid; x < g * D; x += blockDim.x) {
    const int i = x / D, d = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, m_s[v][i]);
    float lsum = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float c = m_s[v][i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_s[v][i] - M);
        lsum += c * l_s[v][i];
        o += c * acc_s[v][i][d];
      }
      o = o / lsum * vscale;
    }
    if (nparts == 1) {
      out[((size_t)s * Hq + hq0 + i) * D + d] = from_f32<QT>(o);
    } else {
      const size_t row = ((size_t)s * Hq + hq0 + i) * a.num_partitions + part;
      a.part_out[row * D + d] = o;
      if (d == 0) {
        a.part_ml[row * 2] = M;
        a.part_ml[row * 2 + 1] = lsum;
      }
    }
  }
}

template <class CT, class QT, int D>
hipError_t launch_g(const DecodeArgs &a, hipStream_t s) {
  const int g = a.num_q_heads / a.cache.num_kv_heads;
  dim3 grid(a.num_partitions, a.cache.num_kv_heads, a.num_seqs), block(256);
  if (g <= 1) decode_valu_kernel<CT, QT, D, 1><<<grid, block, 0, s>>>(a);
  else if (g <= 2) decode_valu_kernel<CT, QT, D, 2><<<grid, block, 0, s>>>(a);
  else if (g <= 4) decode_valu_kernel<CT, QT, D, 4><<<grid, block, 0, s>>>(a);
  else if (g <= 8) decode_valu_kernel<CT, QT, D, 8><<<grid, block, 0, s>>>(a);
  else decode_valu_kernel<CT, QT, D, 16><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <class CT, class QT>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
  return a.cache.head_dim == 64 ? launch_g<CT, QT, 64>(a, s) : launch_g<CT, QT, 128>(a, s);
}

}  // namespace

hipError_t launch_decode_valu(const DecodeArgs &a, hipStream_t s) {
  switch (a.cache.dtype) {
    case kF32: return launch_d<f32_t, f32_t>(a, s);
    case kF16: return launch_d<f16_t, f16_t>(a, s);
    case kBF16: return launch_d<bf16_t, bf16_t>(a, s);
    case kFP8:
      return a.q_dtype == kF16 ? launch_d<fp8_t, f16_t>(a, s) : launch_d<fp8_t, bf16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
