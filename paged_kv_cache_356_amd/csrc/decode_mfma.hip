// decode_mfma.hip — split-K paged decode attention on the matrix cores (MFMA) of gfx950.
//
// Same contract as the vector-ALU kernel: walk each sequence's block table, gather one 16-token
// block of K and V at a time from wherever it landed in the pool ("PagedAttention" (devoured.fyi),
// "PagedAttention in one picture", "Why the attention kernel works at all") and compute ordinary
// softmax(q K^T * scale) V ("Misconceptions": the math is unchanged).  Partitions of
// `partition_size` tokens each give (running max, running sum, normalised output), merged later by
// pa_partition_reduce when a sequence spans more than one.
//
// Why matrix cores: with grouped-query heads the g query heads of one KV head share every K and V
// element, so per 16-token block the work is two small dense products,
//   S^T [16 tokens x 16 heads] = K [16 x D] . Q^T [D x 16 heads]   (g of the 16 head columns real)
//   O^T [D x 16 heads]        += V^T [D x 16 tokens] . P^T [16 tokens x 16 heads]
// On the vector ALUs these cost ~2 fp32 FMAs per KV byte per head, which keeps a wave from issuing
// loads fast enough; on MFMA they take a few hundred cycles per block and the kernel is left bound
// by HBM, which is the point.
//
// Lane layouts (v_mfma_f32_16x16x32_{f16,bf16} and v_mfma_f32_16x16x16{f16,bf16_1k}; lane l,
// c = l % 16, r = l / 16):  A holds row c, reduction indices kpl*r .. kpl*r + kpl-1 (kpl = 8 or 4);
// B holds column c, the same reduction indices; the f32 result holds rows 4r .. 4r+3 of column c.
//  - QK^T: A = K rows (token c), B = Q^T columns (head c).  In the pool layout the 16-byte K vector
//    v of token t sits at vector index v*16 + t, so the 8 dims lane l needs for product kk are the
//    vector (l + 64 kk) of the tile: each load instruction of the wave reads 1 KiB contiguous.
//  - The S^T result gives lane l the scores of tokens 4r..4r+3 for head c: exactly the B operand
//    (P^T, 4 tokens of column c) of the PV product, so probabilities never leave registers.
//  - PV: A = V^T rows (head-dim index 16 nt + c, tokens 4r..4r+3), 4 contiguous elements of the
//    transposed V tile; each load instruction of the wave covers 512 bytes contiguous.
// The softmax state follows the lanes: lane l owns head c; its maximum is uniform over the four
// lanes of column c after two cross-row shuffles.
//
// Probabilities are split p = hi + lo with hi, lo in the MFMA input type, and both parts go through
// the PV product: the result then carries p to ~2^-16 (bf16) or ~2^-22 (f16) relative accuracy, not
// the 2^-8 / 2^-11 of a single rounding.
//
// fp8 (E4M3FN) caches compute in f16: byte c becomes the binary16 with bits
// (c & 0x80) << 8 | (c & 0x7f) << 7, whose value is exactly decode(c) * 2^-8 (normals and
// subnormals alike); the 2^8 goes back into the per-head scales.  The NaN code is mapped to a NaN.
//
// Workgroup = 4 wavefronts for one (partition, KV head, sequence); wavefront w takes the
// partition's blocks w, w+4, ... and keeps the loads of its next blocks in flight while it computes
// the current one.  The four partial states are merged through LDS.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxScanSeqs = 4096;  // persistent grid: sequences whose item prefix fits in LDS
#ifndef PA_DECODE_BUFS
#define PA_DECODE_BUFS 2
#endif
constexpr int kBufs = PA_DECODE_BUFS;  // blocks per wavefront in the load ring
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
#ifndef PA_DECODE_OCC
#define PA_DECODE_OCC 0
#endif

// K/V tiles are read once per decode step: optionally as non-temporal loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <class T> struct NativeVec { using type = T; };
template <> struct NativeVec<uint4> { using type = u32x4_t; };
template <> struct NativeVec<uint2> { using type = u32x2_t; };

template <class T>
__device__ __forceinline__ T load_kv(const char *p) {
  using N = typename NativeVec<T>::type;
  if constexpr (PA_DECODE_NT)
    return __builtin_bit_cast(T, __builtin_nontemporal_load(reinterpret_cast<const N *>(p)));
  else return *reinterpret_cast<const T *>(p);
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

#ifndef PA_FP8_HWCVT
#define PA_FP8_HWCVT 1
#endif
// Scale that the f16 values produced from fp8 codes carry: 2^-8 for the bit mapping below, 1 for
// the hardware conversion.
constexpr float kFp8Unscale = PA_FP8_HWCVT ? 1.0f : 256.0f;

// Four E4M3FN bytes (byte 0 first) -> four binary16 values equal to decode(byte) * 2^-8, or, with
// the hardware conversion (v_cvt_scalef32_pk_f16_fp8 at scale 1), equal to decode(byte).
__device__ __forceinline__ uint2 e4m3x4_to_f16x4(uint32_t x) {
#if PA_FP8_HWCVT
  uint2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true));
  return r;
#else
  const uint32_t t01 = ((x & 0xffu) << 8) | ((x & 0xff00u) << 16);
  const uint32_t t23 = ((x >> 8) & 0xff00u) | (x & 0xff000000u);
  uint2 r;
  r.x = (t01 & 0x80008000u) | ((t01 >> 1) & 0x3f803f80u);
  r.y = (t23 & 0x80008000u) | ((t23 >> 1) & 0x3f803f80u);
  // A byte whose low 7 bits are all ones is the NaN code: give it a binary16 NaN.
  const uint32_t y = x & 0x7f7f7f7fu;
  if (__builtin_expect(((y + 0x01010101u) & 0x80808080u) != 0u, 0)) {
    if ((y & 0x7fu) == 0x7fu) r.x |= 0x7e00u;
    if ((y & 0x7f00u) == 0x7f00u) r.x |= 0x7e000000u;
    if ((y & 0x7f0000u) == 0x7f0000u) r.y |= 0x7e00u;
    if ((y & 0x7f000000u) == 0x7f000000u) r.y |= 0x7e000000u;
  }
  return r;
#endif
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

template <int D>
struct DecodeLds {
  float o[kWaves][D][17];  // each wavefront's unnormalised output, [head-dim][head] (+1 pad)
  float m[kWaves][16];
  float l[kWaves][16];
};

// One work item: partition `part` of sequence s for KV head h, computed by the whole workgroup.
template <class CT, class QT, int D>
__device__ __forceinline__ void decode_item(const DecodeArgs &a, int s_in, int h_in, int part_in,
                                            DecodeLds<D> &lds) {
  // The item is the same for the whole workgroup: keep its coordinates (and so the block-table
  // row and the tile addresses) in scalar registers, which makes the table reads scalar loads.
  const int s = __builtin_amdgcn_readfirstlane(s_in);
  const int h = __builtin_amdgcn_readfirstlane(h_in);
  const int part = __builtin_amdgcn_readfirstlane(part_in);
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;  // fp8 and f16 caches compute in f16
  constexpr int KK = D / 32;                              // QK^T products per block
  using F = Frag<CT, D>;
  constexpr int NT = F::kNT;
  constexpr int kTileBytes = kBlock * D * CT::bytes;
  auto &o_s = lds.o;
  auto &m_s = lds.m;
  auto &l_s = lds.l;

  const int H = a.cache.num_kv_heads, Hq = a.num_q_heads, g = Hq / H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  int Ls = a.context_lens[s];
  Ls = Ls < 0 ? 0 : (Ls > a.max_context_len ? a.max_context_len : Ls);
  const int PT = a.partition_size;
  const int start = part * PT;
  auto *out = static_cast<typename QT::raw *>(a.out);
  if (start >= Ls) {
    if (part == 0) {  // empty context: output is zero
      for (int x = tid; x < g * D; x += blockDim.x)
        out[((size_t)s * Hq + h * g) * D + x] = from_f32<QT>(0.0f);
    }
    return;
  }
  const int end = min(Ls, start + PT);
  const int nparts = (Ls + PT - 1) / PT;

  // Q^T operand: lane l holds head (h*g + col) (zero when col >= g), 8 dims per product kk.  The
  // dims follow the K operand: f16/bf16 tiles give lane group r dims 8r + 32kk; fp8 tiles give
  // 16-byte vectors of 16 dims, split in two products, so dims 16r + 64(kk/2) + 8(kk%2).
  uint4 qop[KK];
  {
    const auto *q = reinterpret_cast<const uint16_t *>(a.q) + (size_t)s * a.q_stride +
                    (size_t)(h * g + col) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int d0 = kFP8 ? 16 * grp + 64 * (kk >> 1) + 8 * (kk & 1) : 8 * grp + 32 * kk;
      qop[kk] = col < g ? *reinterpret_cast<const uint4 *>(q + d0) : make_uint4(0, 0, 0, 0);
    }
  }

  float kscale = a.scale * kLog2e, vscale = 1.0f;
  if constexpr (kFP8) {
    kscale *= a.cache.k_scale[h] * kFp8Unscale;
    vscale = a.cache.v_scale[h] * kFp8Unscale;
  }
  const char *kpool = static_cast<const char *>(a.cache.k_pool);
  const char *vpool = static_cast<const char *>(a.cache.v_pool);
  const int32_t *table = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int nb = a.cache.num_blocks;

  auto load = [&](int bid, F &f) {
    const size_t tile = ((size_t)bid * H + h) * kTileBytes;
    const char *kt = kpool + tile;
    const char *vt = vpool + tile;
#pragma unroll
    for (int i = 0; i < F::kKLoads; ++i)
      f.k[i] = load_kv<uint4>(kt + (size_t)(lane + 64 * i) * 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      f.v[nt] = load_kv<typename F::VRaw>(vt + (size_t)((16 * nt + col) * kBlock + 4 * grp) * CT::bytes);
  };

  // Running maximum (base-2 logits) per head; it starts at a finite floor so that a block whose
  // tokens are all masked gives probabilities exp2(-inf - m) = 0 rather than NaN.
  float m = kNoMax, l = 0.0f;
  f4_t acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Block at token tok0; tokens at or past `lim` are masked (lim = tok0 masks the whole block, for
  // a ring slot that holds no block of this partition).
  auto compute = [&](const F &f, int tok0, int lim) {
    // ---- S^T = K Q^T: lane holds the scores of tokens tok0 + 4 grp + i for head col
    f4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (kFP8) {
#pragma unroll
      for (int i = 0; i < F::kKLoads; ++i) {
        const uint2 a0 = e4m3x4_to_f16x4(f.k[i].x), a1 = e4m3x4_to_f16x4(f.k[i].y);
        const uint2 a2 = e4m3x4_to_f16x4(f.k[i].z), a3 = e4m3x4_to_f16x4(f.k[i].w);
        st = mma_k32<false>(make_uint4(a0.x, a0.y, a1.x, a1.y), qop[2 * i], st);
        st = mma_k32<false>(make_uint4(a2.x, a2.y, a3.x, a3.y), qop[2 * i + 1], st);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) st = mma_k32<kBF>(f.k[kk], qop[kk], st);
    }
    const int t0 = tok0 + 4 * grp;
    float z[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = t0 + i < lim ? st[i] * kscale : -INFINITY;  // select: tail slots never leak
      mx = fmaxf(mx, z[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescaling: the running maximum of a head moves only when a block's maximum exceeds it
    // by more than kSlack (base 2), so probabilities stay below 2^kSlack and the accumulator is
    // rescaled on a few blocks instead of every one.  The first block always moves it (m = -inf).
    const bool grow = mx > m + kSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform branch
      const float mn = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first block, else <= 1
      l *= alpha;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
      m = mn;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(z[i] - m);
    l += (p[0] + p[1]) + (p[2] + p[3]);
    uint2 phi, plo;
    phi.x = pack2<kBF>(p[0], p[1]);
    phi.y = pack2<kBF>(p[2], p[3]);
    plo.x = pack2<kBF>(p[0] - unpack_lo<kBF>(phi.x), p[1] - unpack_hi<kBF>(phi.x));
    plo.y = pack2<kBF>(p[2] - unpack_lo<kBF>(phi.y), p[3] - unpack_hi<kBF>(phi.y));

    // ---- O^T += V^T P^T; V elements of tail tokens are zeroed (select), so NaN there cannot leak
    const bool tail = tok0 + kBlock > lim;  // wave-uniform
    const uint32_t keep0 = (t0 + 0 < lim ? 0xffffu : 0u) | (t0 + 1 < lim ? 0xffff0000u : 0u);
    const uint32_t keep1 = (t0 + 2 < lim ? 0xffffu : 0u) | (t0 + 3 < lim ? 0xffff0000u : 0u);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      uint2 vop;
      if constexpr (kFP8) vop = e4m3x4_to_f16x4(f.v[nt]);
      else vop = f.v[nt];
      if (tail) {
        vop.x &= keep0;
        vop.y &= keep1;
      }
      const f4_t c = mma_k16<kBF>(vop, phi, acc[nt]);
      acc[nt] = mma_k16<kBF>(vop, plo, c);
    }
  };

  // ---- the partition's blocks w, w + 4, ... through a ring of kBufs fragments: while one block
  // is computed, the loads of the next kBufs - 1 blocks of this wavefront are in flight.  Buffer
  // indices are compile-time constants (the inner loop is unrolled), so the ring needs no copies.
  // Every ring slot is loaded and computed on every round, with no branch around either, so each
  // compute waits only for its own slot and the accumulators stay in place: a slot past the end of
  // the range, or whose table entry lies outside the pool, reads tile (0, h) instead (a few
  // L2-resident lines) and is computed with all of its tokens masked, which leaves the state
  // unchanged (its V elements are zeroed by selection, its probabilities are 0).
  const int jb0 = start / kBlock, jb1 = (end + kBlock - 1) / kBlock;
  F buf[kBufs];
  bool ok[kBufs];
#pragma unroll
  for (int b = 0; b < kBufs; ++b) {
    const int j = jb0 + w + b * kWaves;
    const int bid = j < jb1 ? table[j] : -1;
    ok[b] = (unsigned)bid < (unsigned)nb;  // an entry outside the pool is never dereferenced
    load(ok[b] ? bid : 0, buf[b]);
  }
  for (int jr = jb0 + w; jr < jb1; jr += kBufs * kWaves) {
#pragma unroll
    for (int b = 0; b < kBufs; ++b) {
      const int j = jr + b * kWaves;
      compute(buf[b], j * kBlock, ok[b] ? end : j * kBlock);  // branch-free: see the ring note
      const int jn = j + kBufs * kWaves;
      const int bid = jn < jb1 ? table[jn] : -1;
      ok[b] = (unsigned)bid < (unsigned)nb;
      load(ok[b] ? bid : 0, buf[b]);
    }
  }

  // ---- merge the four wavefronts through LDS
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (grp == 0) {
    m_s[w][col] = m;
    l_s[w][col] = l;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) o_s[w][16 * nt + 4 * grp + i][col] = acc[nt][i];
  __syncthreads();

  const int hq0 = h * g;
  for (int x = tid; x < g * D; x += blockDim.x) {
    const int i = x / D, d = x % D;
    float M = kNoMax;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, m_s[v][i]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float c = __builtin_amdgcn_exp2f(m_s[v][i] - M);  // an idle wavefront has l = 0
      lsum += c * l_s[v][i];
      o += c * o_s[v][d][i];
    }
    o = lsum > 0.0f ? o / lsum * vscale : 0.0f;  // no position at all: zero
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

// Grid modes.  Direct: one workgroup per (partition, KV head, sequence) of the launch bounds, the
// ones past a sequence's end returning at once.  Persistent: as many workgroups as fit on the
// device at once, each taking items f = blockIdx.x, + gridDim.x, ... of the flat list of the
// batch's real items, ordered (sequence, partition, KV head) with the KV head fastest; the list
// is the prefix sum of the sequences' partition counts, computed by every workgroup in LDS (an
// empty sequence counts one item, which writes its zero output).  Item sizes are all one
// partition except each sequence's last, so the round-robin split stays balanced without the
// idle workgroups of the direct grid.
template <class CT, class QT, int D>
__global__ __launch_bounds__(256)
#if PA_DECODE_OCC
__attribute__((amdgpu_waves_per_eu(PA_DECODE_OCC, PA_DECODE_OCC)))
#endif
void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeLds<D> lds;
  if (!a.persistent) {
    decode_item<CT, QT, D>(a, blockIdx.z, blockIdx.y, blockIdx.x, lds);
    return;
  }
  __shared__ int prefix[kMaxScanSeqs + 1];
  __shared__ int wave_tot[kWaves];
  const int S = a.num_seqs, H = a.cache.num_kv_heads, PT = a.partition_size;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // thread t counts the items of sequences [t * per, (t + 1) * per)
  const int per = (S + 255) / 256;
  const int s0 = tid * per;
  int mine = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < S) {
      int L = a.context_lens[s];
      L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
      mine += L > 0 ? (L + PT - 1) / PT : 1;
    }
  }
  int incl = mine;  // inclusive scan over the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int v = 0; v < wv; ++v) run += wave_tot[v];
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < S) {
      prefix[s] = run;
      int L = a.context_lens[s];
      L = L < 0 ? 0 : (L > a.max_context_len ? a.max_context_len : L);
      run += L > 0 ? (L + PT - 1) / PT : 1;
    }
  }
  if (tid == 255) prefix[S] = run;  // thread 255 holds the grand total (its chunk ends at S or later)
  __syncthreads();
  const int total = prefix[S] * H;
  for (int f = blockIdx.x; f < total; f += gridDim.x) {
    const int pf = f / H, h = f - pf * H;
    int lo = 0, hi = S - 1;  // largest s with prefix[s] <= pf
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= pf) lo = mid;
      else hi = mid - 1;
    }
    decode_item<CT, QT, D>(a, lo, h, pf - prefix[lo], lds);
    __syncthreads();  // the next item reuses the LDS merge buffers
  }
}

// Workgroups of one instantiation that fit on the device at once (occupancy x compute units),
// looked up once per device.
template <class CT, class QT, int D>
int resident_groups() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int occ = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, decode_mfma_kernel<CT, QT, D>, 256, 0) !=
          hipSuccess || occ < 1)
    occ = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                     hipSuccess || cus < 1)
    cus = 1;
  const int n = occ * cus;
  if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <class CT, class QT, int D>
hipError_t launch_dd(DecodeArgs a, hipStream_t s) {
  const int64_t direct = (int64_t)a.num_partitions * a.cache.num_kv_heads * a.num_seqs;
  a.persistent = a.num_seqs <= kMaxScanSeqs;
  dim3 grid(a.num_partitions, a.cache.num_kv_heads, a.num_seqs);
  if (a.persistent) grid = dim3((unsigned)std::min<int64_t>(direct, resident_groups<CT, QT, D>()));
  decode_mfma_kernel<CT, QT, D><<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <class CT, class QT>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
  return a.cache.head_dim == 64 ? launch_dd<CT, QT, 64>(a, s) : launch_dd<CT, QT, 128>(a, s);
}

}  // namespace

bool decode_mfma_supports(const DecodeArgs &a) {
  const int cdt = a.cache.dtype, qdt = a.q_dtype;
  const bool types = (cdt == kF16 && qdt == kF16) || (cdt == kBF16 && qdt == kBF16) ||
                     (cdt == kFP8 && qdt == kF16);
  const int g = a.num_q_heads / a.cache.num_kv_heads;
  // the Q^T operand is read as 16-byte vectors of 8 elements
  const bool q_aligned = (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0 && a.q_stride % 8 == 0;
  // an empty pool has no tile for the ring's idle slots to read
  return types && g >= 1 && g <= 16 && (a.cache.head_dim == 64 || a.cache.head_dim == 128) &&
         q_aligned && a.cache.num_blocks > 0;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
  switch (a.cache.dtype) {
    case kF16: return launch_d<f16_t, f16_t>(a, s);
    case kBF16: return launch_d<bf16_t, bf16_t>(a, s);
    case kFP8: return launch_d<fp8_t, f16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
