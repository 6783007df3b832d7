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
// the 2^-8 / 2^-11 of a single rounding.  (Measured on MI355X: a single rounding is not faster on
// any workload, the fp8 28-layer batch 2% slower, and its errors are several times larger.)
//
// fp8 (E4M3FN) caches compute in f16: the hardware conversion widens four codes to their exact
// binary16 values (every E4M3FN value is one), the per-head scales multiplying the logits (K) and
// the output (V).
//
// Work items: a wavefront takes one (sequence, partition, KV head) at a time and streams the
// partition's blocks through a ring of register fragments, keeping the loads of its next blocks in
// flight while it computes the current one; its result goes to the output, or to the workspace as
// a partial for pa_partition_reduce.  A shared prefix is computed once for the whole batch by
// workgroup-wide groups of 64 rows that stage each block in LDS.
#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "mfma_common.h"
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kMaxScanSeqs = 4096;  // persistent grid: sequences whose item prefix fits in LDS
// The shared-prefix instantiation also holds the prefix groups' block stages in LDS; its scan
// arrays are halved so that three workgroups still fit on a compute unit.
constexpr int kMaxScanSeqsPrefix = 2048;
// 16-row tiles per wavefront in a prefix group: each block staged in LDS serves 16 kPrefixTiles
// rows per wavefront (two tiles spill registers at three workgroups per compute unit).
constexpr int kPrefixTiles = 1;
// Blocks in flight per wavefront in the ring: two 16-bit fragments, or three fp8 ones (half the
// registers each).  Deeper rings at fewer wavefronts per SIMD measured slower.
constexpr int kDecodeBufs = 2;
constexpr int kFp8Bufs = 3;
// K/V tiles of the sequences' own blocks are read once per call: non-temporal loads.
constexpr bool kDecodeNT = true;
// Wavefronts per SIMD the instantiations are built for (registers capped at 512 / occupancy): three
// (168 registers); the plain decode's fused-append instantiation two (256 registers, no spills),
// measured level with the plain decode on the 32K batch and faster than three on the others; the
// shared-prefix one keeps three (its grid needs three workgroups per compute unit).
constexpr int kDecodeOcc = 3;
constexpr int kAppendOcc = 2;
// Paired items run one wavefront per SIMD (pair_items), so their instantiation can take 256
// registers: the first partition's row state, held until the ring ends, fits without scratch.
constexpr int kPairOcc = 2;

// off: per-lane byte offset; soff: a wave-uniform byte offset added to it.
template <class T, bool kNT>
__device__ __forceinline__ T load_kv(__amdgpu_buffer_rsrc_t r, int off, int soff = 0) {
  constexpr int aux = kNT ? 2 : 0;  // 2: nt
  if constexpr (sizeof(T) == 16)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, aux));
  else if constexpr (sizeof(T) == 8)
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, aux));
  else
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, aux));
}

// The K and V tiles of block bid, KV head h, into f; ok = false (no block in this slot) loads zeros
// without reading memory.
template <class CT, int D, bool kNT>
__device__ __forceinline__ void load_block(const DecodeArgs &a, int bid, bool ok, int h,
                                           Frag<CT, D> &f) {
  using F = Frag<CT, D>;
  constexpr int kTileBytes = kBlock * D * CT::bytes;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const size_t tile = ((size_t)(ok ? bid : 0) * a.cache.num_kv_heads + h) * kTileBytes;
  const int n = ok ? kTileBytes : 0;
  const auto rk = tile_rsrc(static_cast<const char *>(a.cache.k_pool) + tile, n);
  const auto rv = tile_rsrc(static_cast<const char *>(a.cache.v_pool) + tile, n);
#pragma unroll
  for (int i = 0; i < F::kKLoads; ++i) f.k[i] = load_kv<uint4, kNT>(rk, (lane + 64 * i) * 16);
#pragma unroll
  for (int nt = 0; nt < F::kNT; ++nt)
    f.v[nt] = load_kv<typename F::VRaw, kNT>(rv, ((16 * nt + col) * kBlock + 4 * grp) * CT::bytes);
}

// Other block sizes.  The ring always advances by one 16-position step (one product's worth);
// a table entry names a block of kB positions, in the layout of include/pa.h with B = kB.
//  - kB = 32: a block is two steps; step `sub` of block bid reads positions 16 sub .. 16 sub + 15
//    of the tile, through the tile's descriptor as for kB = 16.
//  - kB = 8: a step spans two blocks (b0: positions 0..7 of the step, b1: 8..15).  Lanes of the K
//    operand rows c < 8 and of the V operand lane groups 0-1 read b0, the others b1, so the loads go
//    through one descriptor over the whole pool with per-lane offsets; a lane whose block is absent
//    reads past the descriptor's end (zeros, no memory access), and a step with no block at all
//    gets an empty descriptor.
template <int kB>
struct BlockSteps {
  static_assert(kB == 8 || kB == 16 || kB == 32, "block size");
  static constexpr int kChunk = kB == 8 ? 32 : 64;  // ring steps per chunk of table entries
};

// Lane i's entry of the table entries that ring steps [j0, j0 + kn) read (kB = 8 or 32), -1 past
// those that positions below vend need: entries past a sequence's blocks are never read.
template <int kB>
__device__ __forceinline__ int chunk_table_entries(const int32_t *table, int j0, int kn, int vend) {
  const int lane = threadIdx.x & 63;
  const int e0 = kB == 32 ? j0 >> 1 : 2 * j0;
  const int e1 = min(kB == 32 ? (j0 + kn + 1) >> 1 : 2 * (j0 + kn), (vend + kB - 1) / kB);
  return lane < e1 - e0 ? table[e0 + lane] : -1;
}

template <class CT, int D, bool kNT>
__device__ __forceinline__ void load_block32(const DecodeArgs &a, int bid, bool ok, int sub, int h,
                                             Frag<CT, D> &f) {
  using F = Frag<CT, D>;
  constexpr int kTileBytes = 32 * D * CT::bytes;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const size_t tile = ((size_t)(ok ? bid : 0) * a.cache.num_kv_heads + h) * kTileBytes;
  const int n = ok ? kTileBytes : 0;
  const auto rk = tile_rsrc(static_cast<const char *>(a.cache.k_pool) + tile, n);
  const auto rv = tile_rsrc(static_cast<const char *>(a.cache.v_pool) + tile, n);
  // per-lane parts of the offsets, plus wave-uniform ones (the half, the vector / head-dim rows)
  const int koff = (grp * 32 + col) * 16, voff = (col * 32 + 4 * grp) * CT::bytes;
#pragma unroll
  for (int i = 0; i < F::kKLoads; ++i)
    f.k[i] = load_kv<uint4, kNT>(rk, koff, (4 * i * 32 + 16 * sub) * 16);
  // A step reads half of each head dim's 32-position V^T row, so half of every cache line; the
  // other half belongs to the block's other step, issued next: ordinary loads let it find the
  // line in L2 instead of fetching it again.
#pragma unroll
  for (int nt = 0; nt < F::kNT; ++nt)
    f.v[nt] = load_kv<typename F::VRaw, false>(rv, voff, (16 * nt * 32 + 16 * sub) * CT::bytes);
}

// lane_ok: whether this lane's block (of its K row for the scores, of its positions for the
// probabilities, the same one: lanes 0-31 hold positions of b0, 32-63 of b1) is present.
template <class CT, int D, bool kNT>
__device__ __forceinline__ void load_block8(const DecodeArgs &a, int b0, bool ok0, int b1,
                                            bool ok1, int h, Frag<CT, D> &f) {
  using F = Frag<CT, D>;
  constexpr int kTileBytes = 8 * D * CT::bytes;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const uint32_t pool = (uint32_t)((size_t)a.cache.num_blocks * a.cache.num_kv_heads * kTileBytes);
  const uint32_t n = ok0 || ok1 ? pool : 0u;
  const auto rk = tile_rsrc(static_cast<const char *>(a.cache.k_pool), (int)n);
  const auto rv = tile_rsrc(static_cast<const char *>(a.cache.v_pool), (int)n);
  const int H = a.cache.num_kv_heads;
  // K operand row col: block col >> 3, its position col & 7; an absent block reads past the end
  const bool kok = col < 8 ? ok0 : ok1;
  const uint32_t koff =
      kok ? (uint32_t)((col < 8 ? b0 : b1) * H + h) * kTileBytes + (grp * 8 + (col & 7)) * 16
          : pool;
#pragma unroll
  for (int i = 0; i < F::kKLoads; ++i) f.k[i] = load_kv<uint4, kNT>(rk, (int)koff, i * 4 * 8 * 16);
  // V operand lane group grp: positions 4 grp .. 4 grp + 3 of the step, block grp >> 1
  const bool vok = grp < 2 ? ok0 : ok1;
  const uint32_t voff =
      vok ? (uint32_t)((grp < 2 ? b0 : b1) * H + h) * kTileBytes + (col * 8 + 4 * (grp & 1)) * CT::bytes
          : pool;
#pragma unroll
  for (int nt = 0; nt < F::kNT; ++nt)
    f.v[nt] = load_kv<typename F::VRaw, kNT>(rv, (int)voff, 16 * nt * 8 * CT::bytes);
}

// The probabilities of one block for this lane's column, split p = hi + lo in the MFMA input type.
struct BlockP {
  uint2 hi, lo;
};

// First half of a block step: S^T = K Q^T for the block at token tok0, the online-softmax update
// of the state's maximum and sum (rescaling the accumulator when the maximum moves), and the
// probabilities.  Scores of positions at or past `zlim` (per lane) are masked.
template <class CT, int D>
__device__ __forceinline__ BlockP block_scores(const uint4 (&k)[Frag<CT, D>::kKLoads], float kscale,
                                               int tok0, int zlim, RowState<D> &rs_) {
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;  // fp8 and f16 caches compute in f16
  constexpr int KK = D / 32;
  using F = Frag<CT, D>;
  constexpr int NT = F::kNT;
  const int grp = (threadIdx.x & 63) >> 4;
  const auto &qop = rs_.qop;
  float &m = rs_.m;
  float &l = rs_.l;
  auto &acc = rs_.acc;
  // ---- S^T = K Q^T: lane holds the scores of tokens tok0 + 4 grp + i for head col
  f4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kFP8) {
#pragma unroll
    for (int i = 0; i < F::kKLoads; ++i) {
      const uint2 a0 = e4m3x4_to_f16x4(k[i].x), a1 = e4m3x4_to_f16x4(k[i].y);
      const uint2 a2 = e4m3x4_to_f16x4(k[i].z), a3 = e4m3x4_to_f16x4(k[i].w);
      st = mma_k32<false>(make_uint4(a0.x, a0.y, a1.x, a1.y), qop[2 * i], st);
      st = mma_k32<false>(make_uint4(a2.x, a2.y, a3.x, a3.y), qop[2 * i + 1], st);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) st = mma_k32<kBF>(k[kk], qop[kk], st);
  }
  const int t0 = tok0 + 4 * grp;
  float z[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[i] = t0 + i < zlim ? st[i] * kscale : -INFINITY;  // select: tail slots never leak
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
  BlockP r;
  r.hi.x = pack2<kBF>(p[0], p[1]);
  r.hi.y = pack2<kBF>(p[2], p[3]);
  r.lo.x = pack2<kBF>(p[0] - unpack_lo<kBF>(r.hi.x), p[1] - unpack_hi<kBF>(r.hi.x));
  r.lo.y = pack2<kBF>(p[2] - unpack_lo<kBF>(r.hi.y), p[3] - unpack_hi<kBF>(r.hi.y));
  return r;
}

// Second half: O^T += V^T P^T.  V elements of positions at or past `vlim` (wave-uniform) are
// zeroed (select), so NaN there cannot leak.
template <class CT, int D>
__device__ __forceinline__ void block_values(const typename Frag<CT, D>::VRaw (&v)[Frag<CT, D>::kNT],
                                             const BlockP &pr, int tok0, int vlim,
                                             RowState<D> &rs_) {
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;
  constexpr int NT = Frag<CT, D>::kNT;
  const int grp = (threadIdx.x & 63) >> 4;
  const int t0 = tok0 + 4 * grp;
  const bool tail = tok0 + kBlock > vlim;  // wave-uniform
  const uint32_t keep0 = (t0 + 0 < vlim ? 0xffffu : 0u) | (t0 + 1 < vlim ? 0xffff0000u : 0u);
  const uint32_t keep1 = (t0 + 2 < vlim ? 0xffffu : 0u) | (t0 + 3 < vlim ? 0xffff0000u : 0u);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint2 vop;
    if constexpr (kFP8) vop = e4m3x4_to_f16x4(v[nt]);
    else vop = v[nt];
    if (tail) {
      vop.x &= keep0;
      vop.y &= keep1;
    }
    const f4_t c = mma_k16<kBF>(vop, pr.hi, rs_.acc[nt]);
    rs_.acc[nt] = mma_k16<kBF>(vop, pr.lo, c);
  }
}

// One 16-token block at token tok0 into the state.  Scores of positions at or past `zlim` (per
// lane) are masked; V elements of positions at or past `vlim` (wave-uniform) are zeroed.  zlim =
// vlim = tok0 masks the whole block, which leaves the state unchanged.
template <class CT, int D>
__device__ __forceinline__ void block_step(const Frag<CT, D> &f, float kscale, int tok0, int zlim,
                                           int vlim, RowState<D> &rs_) {
  const BlockP pr = block_scores<CT, D>(f.k, kscale, tok0, zlim, rs_);
  block_values<CT, D>(f.v, pr, tok0, vlim, rs_);
}

// An empty asm that reads and writes every register of a fragment: the compiler must wait for the
// fragment's loads before it.
template <class CT, int D>
__device__ __forceinline__ void settle_frag(Frag<CT, D> &f) {
#pragma unroll
  for (int i = 0; i < Frag<CT, D>::kKLoads; ++i)
    asm volatile("" : "+v"(f.k[i].x), "+v"(f.k[i].y), "+v"(f.k[i].z), "+v"(f.k[i].w));
#pragma unroll
  for (int nt = 0; nt < Frag<CT, D>::kNT; ++nt) {
    if constexpr (sizeof(f.v[nt]) == 8) asm volatile("" : "+v"(f.v[nt].x), "+v"(f.v[nt].y));
    else asm volatile("" : "+v"(f.v[nt]));
  }
}

// The ring: blocks j = jb0 .. jb1 - 1 of table row `table`, KV head h, through kBufs fragments.
// While one block is computed, the loads of the next kBufs - 1 are in flight.
// Buffer indices are compile-time constants (the inner loop is unrolled), so the ring needs no
// copies.  The first kBufs slots are loaded unconditionally (a slot past the end through an empty
// descriptor: zeros, no memory access), and in the full rounds every slot is computed and reloaded
// with a real block, with no branch around either, so each compute waits only for its own slot
// (partial s_waitcnt vmcnt) and the accumulators stay in place.  The last one or two rounds are
// straight-line code that computes and reloads only the blocks that exist: a load issued past the
// end would have to complete before its registers are reused after the ring, which costs the
// wavefront a full memory round trip at the end of every item.  A table entry outside the pool is
// loaded through an empty descriptor too and computed fully masked.
// The wavefront's table entries are fetched before its ring starts, one per lane, and read back with
// v_readlane: a table read inside the ring would be a vector load whose result feeds the next
// address, and waiting for it would drain every load in flight.  A wavefront with more than 64
// blocks runs one ring per 64 of them.  The first 64 entries (tbl0, from first_table_entries)
// come from the caller, which can fetch them while the wavefront's previous item streams.
// kPair: after step mid - 1 (mid > 0) the ring calls at_mid(st), which sets the first partition of
// a paired item aside and resets the row state, and streams on without draining.
struct NoMid {
  template <class T>
  __device__ void operator()(T &) const {}
};

template <class CT, int D, bool kNT, int kB, bool kPair = false, class Mid = NoMid>
__device__ __forceinline__ void stream_blocks(const DecodeArgs &a, const int32_t *table, int h,
                                              int jb0, int jb1, int tbl0, int zlim, int vend,
                                              float kscale, RowState<D> &st, int mid = -1,
                                              Mid &&at_mid = Mid{}) {
  using F = Frag<CT, D>;
  // blocks per wavefront in the load ring: fp8 fragments are half the registers of 16-bit ones
  constexpr int kBufs = std::is_same<CT, fp8_t>::value ? kFp8Bufs : kDecodeBufs;
  constexpr int kCS = BlockSteps<kB>::kChunk;
  const int nb = a.cache.num_blocks;
  const int lane = threadIdx.x & 63;
  const int nk = jb1 > jb0 ? jb1 - jb0 : 0;  // this wave's 16-position steps (blocks at kB = 16)
  // One ring over the chunk of kn <= kCS steps starting at step k0, with the chunk's table
  // entries one per lane in tbl.  The first chunk is run on its own, outside the loop over the
  // others, so that its entries (fetched by the caller) need no wait at a loop header.
  auto chunk = [&](int k0, int kn, int tbl) {
    // table entry e of the chunk; the callers keep e < 64 and k < kn wave-uniform
    auto entry = [&](int e) { return __builtin_amdgcn_readlane(tbl, e < 64 ? e : 63); };
    F buf[kBufs];
    bool ok[kBufs];       // the step has a block (kB = 8: at least one of its two)
    bool lane_ok[kBufs];  // kB = 8: this lane's block of the step is present
    auto load = [&](int b, int k) {
      if constexpr (kB == 16) {
        const int bid = k < kn ? entry(k) : -1;
        ok[b] = (unsigned)bid < (unsigned)nb;  // an entry outside the pool is never dereferenced
        load_block<CT, D, kNT>(a, bid, ok[b], h, buf[b]);
      } else if constexpr (kB == 32) {
        const int j = jb0 + k0 + k;  // absolute step: block j / 2, its half j % 2
        const int bid = k < kn ? entry((j >> 1) - ((jb0 + k0) >> 1)) : -1;
        ok[b] = (unsigned)bid < (unsigned)nb;
        load_block32<CT, D, kNT>(a, bid, ok[b], j & 1, h, buf[b]);
      } else {
        const int b0 = k < kn ? entry(2 * k) : -1, b1 = k < kn ? entry(2 * k + 1) : -1;
        const bool ok0 = (unsigned)b0 < (unsigned)nb, ok1 = (unsigned)b1 < (unsigned)nb;
        ok[b] = ok0 || ok1;
        lane_ok[b] = (lane >> 5) ? ok1 : ok0;
        load_block8<CT, D, kNT>(a, b0, ok0, b1, ok1, h, buf[b]);
      }
    };
    auto compute = [&](int b, int k) {
      const int t0 = (jb0 + k0 + k) * kBlock;
      const bool zok = kB == 8 ? lane_ok[b] : ok[b];
      block_step<CT, D>(buf[b], kscale, t0, zok ? zlim : t0, ok[b] ? vend : t0, st);
      if constexpr (kPair) {
        if (k0 + k + 1 == mid) at_mid(st);  // wave-uniform
      }
    };
#pragma unroll
    for (int b = 0; b < kBufs; ++b) load(b, b);  // slots past the end: zeros, no memory access
    int kr = 0;
    for (; kr + 2 * kBufs <= kn; kr += kBufs) {  // full rounds
#pragma unroll
      for (int b = 0; b < kBufs; ++b) {
        compute(b, kr + b);
        load(b, kr + b + kBufs);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t, kr += kBufs) {  // what is left: fewer than 2 kBufs blocks
#pragma unroll
      for (int b = 0; b < kBufs; ++b) {
        if (kr + b < kn) {
          compute(b, kr + b);
          if (kr + b + kBufs < kn) load(b, kr + b + kBufs);
        }
      }
    }
    // A slot the chunk never computed still has its (empty) first load pending: wait for it now,
    // when it is long done, rather than at the next reuse of its registers, where the wait could
    // not be told apart from one for every memory operation issued since.
#pragma unroll
    for (int b = 0; b < kBufs; ++b) settle_frag(buf[b]);
  };
  if (nk > 0) chunk(0, min(kCS, nk), tbl0);
  for (int k0 = kCS; k0 < nk; k0 += kCS) {
    const int kn = min(kCS, nk - k0);
    if constexpr (kB == 16) chunk(k0, kn, lane < kn ? table[jb0 + k0 + lane] : -1);
    else chunk(k0, kn, chunk_table_entries<kB>(table, jb0 + k0, kn, vend));
  }
}

// Scale of a row's partial outputs in the workspace.  With an fp8 cache the f16-query partials
// stay in units of the cache codes (|x| <= 448, so inside fp16's range whatever the head's scale),
// and the partition reduce applies the head's v_scale; otherwise they carry the full scale.
template <class CT, class QT>
__device__ __forceinline__ float partial_vscale(float vscale) {
  if constexpr (std::is_same<CT, fp8_t>::value && std::is_same<QT, f16_t>::value)
    return 1.0f;
  return vscale;
}

// The appended token of sequence s for KV head h (fused append): lane l holds elements 2 l and
// 2 l + 1 of its K and V rows (two 16-bit values in one word; zeros past D / 2), and every lane the
// token's slot.
struct NewToken {
  uint32_t k, v;
  int64_t slot;
};

// The token is copied from memory straight into this wavefront's part of LDS when the item
// starts (buffer loads with the LDS destination: no register holds it while the blocks stream)
// and read back once the ring is done, long after it has landed.
struct NewTokenStage {
  uint32_t k[64], v[64], slot[64];
};

__device__ __forceinline__ PA_LDS NewTokenStage *new_token_stage() {
  __shared__ __attribute__((aligned(16))) NewTokenStage stage[kWaves];
  return (PA_LDS NewTokenStage *)&stage[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
}

template <int D>
__device__ __forceinline__ void stage_new_token(const DecodeArgs &a, int s, int h) {
  const int lane = threadIdx.x & 63;
  PA_LDS NewTokenStage *st = new_token_stage();
  const size_t e = (size_t)h * D;
  const auto rk = tile_rsrc(reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.append_k) +
                                                           (size_t)s * a.append_k_stride + e),
                            2 * D);
  const auto rv = tile_rsrc(reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.append_v) +
                                                           (size_t)s * a.append_v_stride + e),
                            2 * D);
  const auto rs = tile_rsrc(reinterpret_cast<const char *>(a.append_slots + s), 8);
  // lanes past the row (D = 64) or past the slot's two words read zeros through the bounds
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (PA_LDS void *)st->k, 4, 4 * lane, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (PA_LDS void *)st->v, 4, 4 * lane, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (PA_LDS void *)st->slot, 4, 4 * lane, 0, 0, 0);
}

__device__ __forceinline__ NewToken read_new_token() {
  const int lane = threadIdx.x & 63;
  const PA_LDS NewTokenStage *st = new_token_stage();
  NewToken t;
  t.k = st->k[lane];
  t.v = st->v[lane];
  t.slot = (int64_t)(((uint64_t)st->slot[1] << 32) | st->slot[0]);
  return t;
}

// A new token's pair of 16-bit input values in the cache's encoding, as stored by
// reshape_and_cache: a bit copy for 16-bit caches; for fp8, E4M3FN(float(x) / scale) of each, the
// two bytes in the low half.
template <class CT, class QT>
__device__ __forceinline__ uint32_t encode_pair(uint32_t w, float scale) {
  if constexpr (std::is_same<CT, fp8_t>::value) {
    auto widen = [](uint32_t b) {
      if constexpr (std::is_same<QT, bf16_t>::value) return bf16_bits_to_f32((uint16_t)b);
      else return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
    };
    const uint32_t lo = f32_to_e4m3(__fdiv_rn(widen(w & 0xffffu), scale));
    const uint32_t hi = f32_to_e4m3(__fdiv_rn(widen(w >> 16), scale));
    return lo | (hi << 8);
  } else {
    return w;
  }
}

// Where the fused append reads and writes the pools: the fields it needs, loaded after the ring.
struct AppendPools {
  char *k_pool, *v_pool;
  int num_blocks, block_size, num_kv_heads;
};

// The encoded new token into its slot of both pools, as reshape_and_cache writes it: lane l the
// elements 2 l and 2 l + 1 (adjacent in a K vector; two V^T rows).  Bit copies of the encoded
// width, never value conversions.
template <class CT, int D>
__device__ __forceinline__ void store_new_token(const AppendPools &c, int64_t slot, int h,
                                                uint32_t kenc, uint32_t venc) {
  const int lane = threadIdx.x & 63;
  const int B = c.block_size;
  if (2 * lane >= D || slot < 0 || slot >= (int64_t)c.num_blocks * B) return;
  using Lt = Layout<CT::bytes>;
  using U = typename std::conditional<CT::bytes == 1, uint8_t, uint16_t>::type;
  constexpr int kBits = 8 * CT::bytes;
  const int64_t blk = slot / B;
  const int off = (int)(slot % B);
  const size_t tile = Lt::tile(blk, h, c.num_kv_heads, D, B);
  const int i0 = 2 * lane;
  U *kp = reinterpret_cast<U *>(c.k_pool) + tile;
  U *vp = reinterpret_cast<U *>(c.v_pool) + tile;
  if constexpr (CT::bytes == 1) *reinterpret_cast<uint16_t *>(kp + Lt::k_off(off, i0, B)) = (uint16_t)kenc;
  else *reinterpret_cast<uint32_t *>(kp + Lt::k_off(off, i0, B)) = kenc;
  vp[Lt::v_off(off, i0, B)] = (U)venc;
  vp[Lt::v_off(off, i0 + 1, B)] = (U)(venc >> kBits);
}

// Position `off` of block b, KV head h, as the pool holds it, in the word layout of the new token
// (lane l: elements 2 l and 2 l + 1 of K and of V).
template <class CT, int D>
__device__ __forceinline__ void pool_position(const AppendPools &c, int b, int off, int h,
                                              uint32_t &kw, uint32_t &vw) {
  const int lane = threadIdx.x & 63;
  const int B = c.block_size;
  using Lt = Layout<CT::bytes>;
  using U = typename std::conditional<CT::bytes == 1, uint8_t, uint16_t>::type;
  constexpr int kBits = 8 * CT::bytes;
  kw = vw = 0u;
  if (2 * lane >= D) return;
  const size_t tile = Lt::tile(b, h, c.num_kv_heads, D, B);
  const int i0 = 2 * lane;
  const U *kp = reinterpret_cast<const U *>(c.k_pool) + tile;
  const U *vp = reinterpret_cast<const U *>(c.v_pool) + tile;
  if constexpr (CT::bytes == 1) kw = *reinterpret_cast<const uint16_t *>(kp + Lt::k_off(off, i0, B));
  else kw = *reinterpret_cast<const uint32_t *>(kp + Lt::k_off(off, i0, B));
  vw = (uint32_t)vp[Lt::v_off(off, i0, B)] | ((uint32_t)vp[Lt::v_off(off, i0 + 1, B)] << kBits);
}

// The kernel's argument struct read through the kernel-argument segment, its address passed
// through an empty asm: the compiler cannot reuse values loaded before, so the fields the append
// needs after the ring are loaded then, instead of being held in scalar registers while the
// blocks stream.  The struct is the decode kernel's only parameter, at offset 0.
__device__ __forceinline__ const __attribute__((address_space(4))) DecodeArgs *fresh_args() {
  auto *p = (const __attribute__((address_space(4))) DecodeArgs *)
      __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return p;
}

// 16-bit floats (f16, or bf16 when kBF) to fp32.
template <bool kBF>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (kBF) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
}
template <bool kBF>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (kBF) return __uint_as_float(w & 0xffff0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// The fused append's tail, after the ring: position L - 1 is the new token when its slot is in the
// pool (written there now), else what the pool holds at L - 1 (no write).  The position's K and V,
// in the cache's encoding, go back to this wavefront's LDS stage, from which each lane reads the
// dims of its query operand (score) and of its accumulator rows (value); the position enters the
// online softmax in fp32 vector arithmetic, with the ring's lazy-rescaling rule.
template <class CT, class QT, int D>
__device__ __forceinline__ void append_tail(int rs, int h, int L, float kscale, RowState<D> &st) {
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;  // fp8 caches compute in f16
  const int lane = threadIdx.x & 63, grp = lane >> 4;
  // The compiler does not order the copies into LDS before these reads: wait for them here, where
  // the ring has drained (an item without blocks waits for the copies themselves).
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const auto *ka = fresh_args();
  AppendPools c;
  c.k_pool = static_cast<char *>(ka->cache.k_pool);
  c.v_pool = static_cast<char *>(ka->cache.v_pool);
  c.num_blocks = ka->cache.num_blocks;
  c.block_size = ka->cache.block_size;
  c.num_kv_heads = ka->cache.num_kv_heads;
  PA_LDS NewTokenStage *sg = new_token_stage();
  const NewToken nt = read_new_token();
  const int64_t aslot =
      (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(nt.slot >> 32)) << 32) |
                (uint32_t)__builtin_amdgcn_readfirstlane((int)nt.slot));
  const bool write = aslot >= 0 && aslot < (int64_t)c.num_blocks * c.block_size;
  uint32_t kenc = 0u, venc = 0u;
  bool have = write;
  if (write) {
    float ks = 1.0f, vs = 1.0f;
    if constexpr (kFP8) {
      using cfloat = const __attribute__((address_space(4))) float;
      ks = ((cfloat *)(uintptr_t)ka->cache.k_scale)[h];
      vs = ((cfloat *)(uintptr_t)ka->cache.v_scale)[h];
    }
    kenc = encode_pair<CT, QT>(nt.k, ks);
    venc = encode_pair<CT, QT>(nt.v, vs);
  } else if (L > 0) {
    const int p = L - 1, B = c.block_size;
    const int32_t *table = ka->block_tables + (size_t)rs * ka->max_blocks_per_seq;
    const int b = __builtin_amdgcn_readfirstlane(table[p / B]);
    have = (unsigned)b < (unsigned)c.num_blocks;  // an entry outside the pool: left out
    if (have) pool_position<CT, D>(c, b, p % B, h, kenc, venc);
  }
  if (have && L > 0) {
    // the encoded position, dims contiguous (lanes past D / 2 hold zeros)
    if constexpr (kFP8) {
      ((PA_LDS uint16_t *)sg->k)[lane] = (uint16_t)kenc;
      ((PA_LDS uint16_t *)sg->v)[lane] = (uint16_t)venc;
    } else {
      sg->k[lane] = kenc;
      sg->v[lane] = venc;
    }
    const PA_LDS char *kb = (const PA_LDS char *)sg->k;
    const PA_LDS char *vb = (const PA_LDS char *)sg->v;
    // score: this lane's 8 query dims per product kk, summed over the four lane groups
    float z = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const int d0 = kFP8 ? 16 * grp + 64 * (kk >> 1) + 8 * (kk & 1) : 8 * grp + 32 * kk;
      uint4 kv;
      if constexpr (kFP8) {
        const uint2 b8 = lds_load<uint2>(kb + d0);
        const uint2 a = e4m3x4_to_f16x4(b8.x), b = e4m3x4_to_f16x4(b8.y);
        kv = make_uint4(a.x, a.y, b.x, b.y);
      } else {
        kv = lds_load<uint4>(kb + 2 * d0);
      }
      const uint4 q = st.qop[kk];
      z += half_lo<kBF>(q.x) * half_lo<kBF>(kv.x) + half_hi<kBF>(q.x) * half_hi<kBF>(kv.x);
      z += half_lo<kBF>(q.y) * half_lo<kBF>(kv.y) + half_hi<kBF>(q.y) * half_hi<kBF>(kv.y);
      z += half_lo<kBF>(q.z) * half_lo<kBF>(kv.z) + half_hi<kBF>(q.z) * half_hi<kBF>(kv.z);
      z += half_lo<kBF>(q.w) * half_lo<kBF>(kv.w) + half_hi<kBF>(q.w) * half_hi<kBF>(kv.w);
    }
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    z *= kscale;
    const bool grow = z > st.m + kSlack;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform branch
      const float mn = grow ? z : st.m;
      const float alpha = __builtin_amdgcn_exp2f(st.m - mn);
      st.l *= alpha;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) st.acc[t] *= alpha;
      st.m = mn;
    }
    const float pr = __builtin_amdgcn_exp2f(z - st.m);
    if (grp == 0) st.l += pr;  // the row's sum adds the four lane groups at the end
    // value: accumulator rows 16 t + 4 grp + i of this lane's column
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int d = 16 * t + 4 * grp;
      uint2 vv;
      if constexpr (kFP8) vv = e4m3x4_to_f16x4(lds_load<uint32_t>(vb + d));
      else vv = lds_load<uint2>(vb + 2 * d);
      st.acc[t][0] += pr * half_lo<kBF>(vv.x);
      st.acc[t][1] += pr * half_hi<kBF>(vv.x);
      st.acc[t][2] += pr * half_lo<kBF>(vv.y);
      st.acc[t][3] += pr * half_hi<kBF>(vv.y);
    }
  }
  // the persistent grid leaves the writes to write_token_rows
  if (write && !ka->persistent) store_new_token<CT, D>(c, aslot, h, kenc, venc);
}

// Fused append on the persistent grid: the new tokens' writes into the pools, row (s, h) by the
// wavefront of rank GW - 1 - (s H + h) mod GW once its items are done.  The high ranks are those
// with fewest or no items, so the stores (2- and 4-byte pieces over ~80 cache lines per row) stay
// off the item streams; the rows' last items attend to the token from their own copy, and their
// walk never reads its position, so nothing waits for these writes.
template <class CT, class QT, int D>
__device__ __forceinline__ void write_token_rows(const DecodeArgs &a, int rank, int GW) {
  const int lane = threadIdx.x & 63;
  const int H = a.cache.num_kv_heads, rows = a.num_seqs * H;
  AppendPools c;
  c.k_pool = static_cast<char *>(a.cache.k_pool);
  c.v_pool = static_cast<char *>(a.cache.v_pool);
  c.num_blocks = a.cache.num_blocks;
  c.block_size = a.cache.block_size;
  c.num_kv_heads = H;
  for (int r = GW - 1 - rank; r < rows; r += GW) {
    const int s = r / H, h = r - (r / H) * H;
    // with a shared prefix, a context that does not extend past it takes no write (its position
    // would lie in the prefix's blocks, which every sequence of the batch reads)
    if (a.append_from > 0 && __builtin_amdgcn_readfirstlane(clamp_len(a, s)) <= a.append_from)
      continue;
    const int64_t slot = a.append_slots[s];
    const int64_t sl =
        (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(slot >> 32)) << 32) |
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)slot));
    if (sl < 0 || sl >= (int64_t)c.num_blocks * c.block_size) continue;
    uint32_t kw = 0u, vw = 0u;
    if (2 * lane < D) {
      const size_t e = (size_t)h * D + 2 * lane;
      kw = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.append_k) +
                                               (size_t)s * a.append_k_stride + e);
      vw = *reinterpret_cast<const uint32_t *>(static_cast<const uint16_t *>(a.append_v) +
                                               (size_t)s * a.append_v_stride + e);
    }
    float ks = 1.0f, vs = 1.0f;
    if constexpr (std::is_same<CT, fp8_t>::value) {
      using cfloat = const __attribute__((address_space(4))) float;
      ks = ((cfloat *)(uintptr_t)a.cache.k_scale)[h];
      vs = ((cfloat *)(uintptr_t)a.cache.v_scale)[h];
    }
    store_new_token<CT, D>(c, sl, h, encode_pair<CT, QT>(kw, ks), encode_pair<CT, QT>(vw, vs));
  }
}

// ---------------------------------------------------------------------------------------------
// The work of one wavefront: KV head h over blocks [jb0, jb1) of `table`, against up to 16 query
// rows (the 16 columns of the products).  This lane's column is query row (rs, rhq) (query row rs
// at q_stride, head rhq; output row rs * Hq + rhq), or padding when !rvalid; positions at or past
// its `lim` are masked, and V elements of positions at or past `end` (wave-uniform) are zeroed.
// The result goes to workspace partition `slot`, or straight to the output when slot < 0.
// kNT: read K/V with non-temporal loads (each tile is read once per call), or with ordinary loads
// (tiles that other wavefronts of the call read too).  tbl0: lane i's entry of the first 64
// blocks (first_table_entries).  settle: a value whose load is in flight (the next item's first
// table entries), waited for once this item's blocks are done.
// kPair: the blocks are two partitions, the first mid steps long (mid > 0); its state is set aside
// when the ring passes into the second, and its partial goes to workspace slot mid_slot after.
template <class CT, class QT, int D, bool kNT, int kB, bool kPair = false>
__device__ __forceinline__ void rows_core(const DecodeArgs &a, const int32_t *table, int h,
                                          int jb0, int jb1, int end, int slot, int rs, int rhq,
                                          bool rvalid, int lim, int tbl0, int &settle, bool append,
                                          int L, int mid = -1, int mid_slot = -1) {
  RowState<D> st;
  load_query<CT, D>(a, rs, rhq, rvalid, st);
  if (append) stage_new_token<D>(a, rs, h);
  float kscale, vscale;
  head_scales<CT>(a, h, kscale, vscale);
  // Paired items: at the boundary the first partition's state moves to `first` (its partial is
  // stored after the ring: a store inside it measured 5 us slower on the 32K batch) and the row
  // state starts over.
  RowState<D> first;
  if constexpr (kPair) {
    first.m = kNoMax;
    first.l = 0.0f;
    auto at_mid = [&](RowState<D> &r) {
      first.m = r.m;
      first.l = r.l;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        first.acc[nt] = r.acc[nt];
        r.acc[nt] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
      r.m = kNoMax;
      r.l = 0.0f;
    };
    stream_blocks<CT, D, kNT, kB, true>(a, table, h, jb0, jb1, tbl0, lim, end, kscale, st, mid,
                                        at_mid);
  } else {
    stream_blocks<CT, D, kNT, kB>(a, table, h, jb0, jb1, tbl0, lim, end, kscale, st);
  }
  // Fused append (wave-uniform): position L - 1 was left out of the ring; it is the new token when
  // the slot is in the pool, else what the pool holds there (no write).
  if (append) append_tail<CT, QT, D>(rs, h, L, kscale, st);
  // Wait here, where the ring has nothing left in flight, for every load this item started that its
  // blocks may not have consumed (the query and table entries of an item without blocks) and for
  // `settle` (the next item's table entries, fetched before this item started): later, behind this
  // item's stores, such a wait could not be told apart from a wait for the stores themselves.
  asm volatile("" : "+v"(settle), "+v"(tbl0));
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    asm volatile("" : "+v"(st.qop[kk].x), "+v"(st.qop[kk].y), "+v"(st.qop[kk].z), "+v"(st.qop[kk].w));
  emit_rows<QT, D>(a, st, vscale, partial_vscale<CT, QT>(vscale), slot, rs, rhq, rvalid);
  if constexpr (kPair)
    if (mid > 0)
      emit_rows<QT, D>(a, first, vscale, partial_vscale<CT, QT>(vscale), mid_slot, rs, rhq, rvalid);
}

// Wavefront item of the decode: KV head h over positions [jb0 * 16, end) of sequence s's block
// table row, against the g query heads of s (columns 0 .. g - 1 of the products).  Wavefronts of
// one workgroup run their items independently, so one wavefront's item prologue (query, table
// fetch, first loads) and epilogue overlap the other wavefronts' block streams.
template <class CT, class QT, int D, bool kNT, int kB, bool kApp, bool kPair = false>
__device__ __forceinline__ void wave_item(const DecodeArgs &a, int s_in, int h_in, int jb0_in,
                                          int jb1_in, int end_in, int slot_in, int L_in, int tbl0,
                                          int &settle, int mid_in = -1, int mid_slot_in = -1) {
  // The item is the same for the whole wavefront: keep its fields (and so the tile addresses) in
  // scalar registers.
  const int s = __builtin_amdgcn_readfirstlane(s_in);
  const int h = __builtin_amdgcn_readfirstlane(h_in);
  const int jb0 = __builtin_amdgcn_readfirstlane(jb0_in);
  const int jb1 = __builtin_amdgcn_readfirstlane(jb1_in);
  const int end = __builtin_amdgcn_readfirstlane(end_in);
  const int slot = __builtin_amdgcn_readfirstlane(slot_in);
  const int g = a.num_q_heads / a.cache.num_kv_heads;
  const int col = threadIdx.x & 15;
  const bool rvalid = col < g;
  const int rhq = h * g + (rvalid ? col : 0);
  const int32_t *table = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  // Fused append: the row's last item (the one whose positions end at the context length) writes
  // the new token and takes position L - 1 from registers; its pool walk stops before it.
  const int L = __builtin_amdgcn_readfirstlane(L_in);
  const bool append = kApp && end == L && !(a.append_from > 0 && L <= a.append_from);
  const int e = append && L > 0 ? L - 1 : end;
  rows_core<CT, QT, D, kNT, kB, kPair>(
      a, table, h, jb0, append ? min(jb1, (e + kBlock - 1) / kBlock) : jb1, e, slot, s, rhq,
      rvalid, e, tbl0, settle, append, L, __builtin_amdgcn_readfirstlane(mid_in),
      __builtin_amdgcn_readfirstlane(mid_slot_in));
}

// ---------------------------------------------------------------------------------------------
// Prefix groups through LDS.  The four wavefronts of a workgroup take 64 flat rows of one KV head
// over the same blocks of the shared prefix, so each block is fetched once per workgroup: every
// wavefront copies its share of the block's K and V tiles straight into an LDS stage (buffer loads
// with the LDS destination, no registers), the workgroup meets at a barrier, and each wavefront
// reads the whole block back from LDS into the fragment layout of the register ring.  kStages
// stages keep kStages - 1 blocks in flight while one is computed.  Each stage is a variable of its
// own, so the compiler can tell a read of one stage from the copies still landing in the others.

template <class CT, int D>
struct PrefixStages {
  static constexpr int kTileBytes = kBlock * D * CT::bytes;
  static constexpr int kBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kChunks = kBytes / 1024;  // 1 KiB copies (64 lanes x 16 bytes) per block
  static constexpr int kPerWave = (kChunks + kWaves - 1) / kWaves;
  static constexpr int kStages = kBytes >= 8192 ? 4 : 8;
  static_assert(kChunks >= 2 && (kChunks % kWaves == 0 || kChunks < kWaves), "stage split");
};

// This wavefront's share of the K and V tiles of block bid (KV head h) into stage I; a slot
// without a block (ok = false) copies through an empty descriptor and touches no memory.
template <class CT, int D, int I>
__device__ __forceinline__ void stage_block(const DecodeArgs &a, int bid, bool ok, int h) {
  using P = PrefixStages<CT, D>;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const size_t tile = ((size_t)(ok ? bid : 0) * a.cache.num_kv_heads + h) * P::kTileBytes;
  const int n = ok ? P::kTileBytes : 0;
  const auto rk = tile_rsrc(static_cast<const char *>(a.cache.k_pool) + tile, n);
  const auto rv = tile_rsrc(static_cast<const char *>(a.cache.v_pool) + tile, n);
  auto *stage = prefix_stage<P::kBytes, I>();
#pragma unroll
  for (int i = 0; i < P::kPerWave; ++i) {
    const int c = w + kWaves * i;  // 1 KiB chunk of the stage
    if (P::kChunks % kWaves == 0 || c < P::kChunks) {
      const bool v = c * 1024 >= P::kTileBytes;
      const int off = c * 1024 - (v ? P::kTileBytes : 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(v ? rv : rk,
                                               (PA_LDS void *)(stage + c * 1024),
                                               16, off + 16 * lane, 0, 0, 0);
    }
  }
}

// The K and V tiles of stage I into registers, at the offsets load_block reads them at.
template <class CT, int D, int I, int N>
__device__ __forceinline__ void read_stage_k(uint4 (&k)[N]) {
  static_assert(N == Frag<CT, D>::kKLoads, "K fragment");
  using P = PrefixStages<CT, D>;
  const int lane = threadIdx.x & 63;
  const auto *stage = prefix_stage<P::kBytes, I>();
#pragma unroll
  for (int i = 0; i < N; ++i) k[i] = lds_load<uint4>(stage + (lane + 64 * i) * 16);
}

template <class CT, int D, int I, class VR, int N>
__device__ __forceinline__ void read_stage_v(VR (&v)[N]) {
  static_assert(N == Frag<CT, D>::kNT, "V fragment");
  using P = PrefixStages<CT, D>;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const auto *stage = prefix_stage<P::kBytes, I>();
#pragma unroll
  for (int nt = 0; nt < N; ++nt)
    v[nt] = lds_load<VR>(stage + P::kTileBytes + ((16 * nt + col) * kBlock + 4 * grp) * CT::bytes);
}

// Prefix group: kPrefixTiles tiles of 16 flat rows per wavefront, wavefront w taking rows
// row0 + 16 kPrefixTiles w .. (flat row r is query head h*g + r % g of sequence r / g; rows past
// the batch are padding), all over prefix blocks [jb0, jb1), jb1 - jb0 <= 64, whose ids are lane
// i's `tbl` (first_table_entries).  The whole workgroup calls this with the same arguments; each
// block read from LDS serves all of the wavefront's tiles.  Each row masks the positions at or
// past its own context length (`lens`).
template <class CT, class QT, int D>
__device__ __forceinline__ void prefix_group(const DecodeArgs &a, const int *lens, int h_in,
                                             int row0_in, int jb0_in, int jb1_in, int end_in,
                                             int slot_in, int tbl) {
  using P = PrefixStages<CT, D>;
  constexpr int kS = P::kStages;
  constexpr int kT = kPrefixTiles;
  const int h = __builtin_amdgcn_readfirstlane(h_in);
  const int row0 = __builtin_amdgcn_readfirstlane(row0_in);
  const int jb0 = __builtin_amdgcn_readfirstlane(jb0_in);
  const int jb1 = __builtin_amdgcn_readfirstlane(jb1_in);
  const int end = __builtin_amdgcn_readfirstlane(end_in);
  const int slot = __builtin_amdgcn_readfirstlane(slot_in);
  const int H = a.cache.num_kv_heads, g = a.num_q_heads / H;
  const int col = threadIdx.x & 15;
  RowState<D> st[kT];
  bool rvalid[kT];
  int rs[kT], rhq[kT], lim[kT];
#pragma unroll
  for (int j = 0; j < kT; ++j) {
    const int r = row0 + 16 * j + col;  // past the batch: padding (a whole tile may be padding)
    rvalid[j] = r < a.num_seqs * g;
    rs[j] = rvalid[j] ? r / g : 0;
    rhq[j] = h * g + (rvalid[j] ? r % g : 0);
    lim[j] = rvalid[j] ? min(end, lens[rs[j]]) : end;
    load_query<CT, D>(a, rs[j], rhq[j], rvalid[j], st[j]);
  }
  float kscale, vscale;
  head_scales<CT>(a, h, kscale, vscale);
  const int nb = a.cache.num_blocks;
  const int nk = jb1 - jb0;
  auto issue = [&](auto I, int k) {  // block k into stage I (past the end: an empty copy)
    const int bid = k < nk ? __builtin_amdgcn_readlane(tbl, k < 64 ? k : 63) : -1;
    stage_block<CT, D, decltype(I)::value>(a, bid, (unsigned)bid < (unsigned)nb, h);
  };
  auto step = [&](auto I, int k) {  // compute block k from stage I, refill the previous stage
    constexpr int i = decltype(I)::value;
    stage_barrier<P::kPerWave * (kS - 2)>();  // block k landed for every wavefront
    issue(std::integral_constant<int, (i + kS - 1) % kS>{}, k + kS - 1);
    const int bid = __builtin_amdgcn_readlane(tbl, k < 64 ? k : 63);
    const bool ok = (unsigned)bid < (unsigned)nb;
    const int t0 = (jb0 + k) * kBlock;
    // K for every tile, then V for every tile: one tile's worth of block registers at a time
    BlockP pr[kT];
    {
      uint4 kf[Frag<CT, D>::kKLoads];
      read_stage_k<CT, D, i>(kf);
#pragma unroll
      for (int j = 0; j < kT; ++j) pr[j] = block_scores<CT, D>(kf, kscale, t0, ok ? lim[j] : t0, st[j]);
    }
    typename Frag<CT, D>::VRaw vf[Frag<CT, D>::kNT];
    read_stage_v<CT, D, i>(vf);
#pragma unroll
    for (int j = 0; j < kT; ++j) block_values<CT, D>(vf, pr[j], t0, ok ? end : t0, st[j]);
  };
  // The block ids and the queries arrive before the first copy is issued: a wait for them after it
  // would also wait for the copy.  The stages' previous readers (the workgroup's last block) are
  // done before they are refilled.
  asm volatile("" : "+v"(tbl));
#pragma unroll
  for (int j = 0; j < kT; ++j)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      asm volatile("" : "+v"(st[j].qop[kk].x), "+v"(st[j].qop[kk].y), "+v"(st[j].qop[kk].z),
                   "+v"(st[j].qop[kk].w));
  stage_barrier<63>();
  static_for<0, kS - 1>([&](auto I) { issue(I, decltype(I)::value); });
  // Full rounds run every step without a branch, so the compiler knows at each LDS read which
  // copies are still in flight; the last round (fewer than kS blocks) is guarded.
  int k0 = 0;
  for (; k0 + kS <= nk; k0 += kS) static_for<0, kS>([&](auto I) { step(I, k0 + decltype(I)::value); });
  static_for<0, kS>([&](auto I) {
    if (k0 + decltype(I)::value < nk) step(I, k0 + decltype(I)::value);
  });
#pragma unroll
  for (int j = 0; j < kT; ++j)
    emit_rows<QT, D>(a, st[j], vscale, partial_vscale<CT, QT>(vscale), slot, rs[j], rhq[j],
                     rvalid[j]);
}

// Items of sequence s: plain decode, partitions of its context (an empty context counts one item,
// which writes its zeros); shared-prefix decode, partitions of the positions after the prefix
// (possibly none).
// With paired items, a row's partitions are taken two at a time (the last one alone when odd).
__device__ __forceinline__ int seq_items(const DecodeArgs &a, int L) {
  if (a.prefix_len > 0) return row_partitions(a, L) - a.prefix_chunks;
  if (L <= 0) return 1;
  return a.pair_items ? (row_partitions(a, L) + 1) / 2 : row_partitions(a, L);
}

// Sequence item `part` of sequence s (context length L), KV head h: its blocks [jb0, jb1), the end
// of its positions and its workspace slot (-1: the output itself).  A paired item covers
// partitions 2 part and 2 part + 1: slot is the second's, and the first, mid steps long, goes to
// mid_slot (mid = -1: a single partition).
struct SeqItem {
  int s, h, jb0, jb1, end, slot, L, mid, mid_slot;
};

__device__ __forceinline__ SeqItem sequence_item(const DecodeArgs &a, int s, int L, int part,
                                                 int h) {
  const int PT = a.partition_size;
  SeqItem it{s, h, 0, 0, 0, -1, L, -1, -1};
  int start, end;
  if (a.prefix_len > 0) {
    partition_range(a.prefix_len, L, PT, part, &start, &end);
    it.slot = a.prefix_chunks + part;
  } else if (L > 0 && a.pair_items) {
    const int n = (L + PT - 1) / PT;
    const int p0 = 2 * part, p1 = min(n, p0 + 2);
    int s1, e0;
    partition_range(0, L, PT, p0, &start, &e0);
    partition_range(0, L, PT, p1 - 1, &s1, &end);
    it.slot = L > PT ? p1 - 1 : -1;
    if (p1 - p0 == 2) {
      it.mid = (e0 - start) / kBlock;
      it.mid_slot = p0;
    }
  } else if (L > 0) {
    partition_range(0, L, PT, part, &start, &end);
    it.slot = L > PT ? part : -1;
  } else {  // empty context: no block, zeros written straight to the output
    start = end = 0;
  }
  it.jb0 = start / kBlock;
  it.jb1 = (end + kBlock - 1) / kBlock;
  it.end = end;
  return it;
}

template <class CT, class QT, int D, int kB, bool kApp, bool kPair = false>
__device__ __forceinline__ void run_sequence_item(const DecodeArgs &a, const SeqItem &it, int tbl0,
                                                  int &settle) {
  wave_item<CT, QT, D, kDecodeNT, kB, kApp, kPair>(a, it.s, it.h, it.jb0, it.jb1, it.end, it.slot,
                                                   it.L, tbl0, settle, it.mid, it.mid_slot);
}

// Lane i's table entry of the first ring chunk of a sequence item (the table entries of its first
// 64 blocks at kB = 16).
template <int kB>
__device__ __forceinline__ int item_table_entries(const DecodeArgs &a, const SeqItem &it) {
  const int32_t *row = a.block_tables + (size_t)it.s * a.max_blocks_per_seq;
  if constexpr (kB == 16) return first_table_entries(row, it.jb0, it.jb1);
  else
    return chunk_table_entries<kB>(row, it.jb0, min(BlockSteps<kB>::kChunk, it.jb1 - it.jb0),
                                   it.end);
}

// Grid modes.  Direct (plain decode only, more than kMaxScanSeqs sequences): wavefront
// 4 blockIdx.x + w takes flat item (partition, KV head, sequence) of the launch bounds, the ones
// past a sequence's end returning at once.  Persistent: as many workgroups as fit on the device
// at once, every wavefront taking its share of the sequence items, located through the prefix sum
// of the sequences' item counts that every workgroup computes in LDS.
// With a shared prefix, the prefix is cut into groups of 64 flat rows (sequence, query head) of
// one KV head and chunks of up to kPrefixChunk positions; workgroup b takes groups b, b + G, ...
// (G workgroups), its wavefront w the group's rows 16 w .. 16 w + 15.  The four wavefronts share
// each block through LDS (prefix_group), so a block crosses from L2 once per group instead of once
// per 16 rows.  The sequence items go first to the wavefronts of workgroups without prefix work, so
// the streaming of private blocks from HBM starts at once beside the prefix groups.
template <class CT, class QT, int D, bool kPre, int kB, bool kApp, bool kPair = false>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kPair ? kPairOcc : kApp && !kPre ? kAppendOcc : kDecodeOcc)))
void decode_mfma_kernel(DecodeArgs a) {
  static_assert(!kPre || kB == 16, "the shared prefix runs on 16-position blocks");
  static_assert(!kPair || (!kPre && kB == 16), "paired items: plain decode, 16 positions");
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.num_seqs, H = a.cache.num_kv_heads, g = a.num_q_heads / H;
  const int PT = a.partition_size;
  if (!a.persistent) {
    if constexpr (kPair) return;  // the launcher pairs items only on the persistent grid
    const int64_t f = (int64_t)blockIdx.x * kWaves + w;
    const int part = (int)(f % a.num_partitions);
    const int h = (int)((f / a.num_partitions) % H);
    const int64_t s = f / ((int64_t)a.num_partitions * H);
    if (s >= S) return;
    const int L = clamp_len(a, (int)s);
    const int n = L > 0 ? (L + PT - 1) / PT : 1;
    if (part < n) {
      const SeqItem it = sequence_item(a, (int)s, L, part, h);
      int none = 0;
      run_sequence_item<CT, QT, D, kB, kApp>(a, it, item_table_entries<kB>(a, it), none);
    }
    return;
  }
  constexpr int kScan = kPre ? kMaxScanSeqsPrefix : kMaxScanSeqs;
  static_assert(kScan <= (1 << (32 - kOrderCountBits)), "sequence ids must fit beside the counts");
  // prefix[i]: items of the list entries before entry i; with a dealing order the entry's sequence
  // sits above the count, in bits kOrderCountBits and up (the launcher passes an order only when
  // every count fits below them).
  __shared__ int prefix[kScan + 1];
  __shared__ int lens[kScan];  // clamped context lengths, by sequence
  __shared__ int wave_tot[kWaves];
  // The item list runs over the sequences in batch order, or in the caller's seq_order; an entry
  // of seq_order outside [0, S) contributes no item.  Thread t counts the items of list entries
  // [t * per, (t + 1) * per).
  const int32_t *ord = a.seq_order;
  const int per = (S + 255) / 256;
  const int s0 = tid * per;
  int mine = 0;
  if (ord) {
    for (int i = 0; i < per; ++i)
      if (s0 + i < S) {
        lens[s0 + i] = clamp_len(a, s0 + i);
        prefix[s0 + i] = ord[s0 + i];  // this thread's entries, until their counts replace them
      }
    __syncthreads();
    for (int i = 0; i < per; ++i)
      if (s0 + i < S) {
        const int s = prefix[s0 + i];
        mine += (unsigned)s < (unsigned)S ? seq_items(a, lens[s]) : 0;
      }
  } else {
    for (int i = 0; i < per; ++i)
      if (s0 + i < S) {
        const int L = clamp_len(a, s0 + i);
        lens[s0 + i] = L;
        mine += seq_items(a, L);
      }
  }
  int incl = mine;  // inclusive scan over the wavefront
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int run = incl - mine;
  for (int v = 0; v < w; ++v) run += wave_tot[v];
  for (int i = 0; i < per; ++i) {
    const int j = s0 + i;
    if (j < S) {
      if (ord) {
        const int s = prefix[j];
        const bool valid = (unsigned)s < (unsigned)S;
        prefix[j] = run | (int)((unsigned)(valid ? s : 0) << kOrderCountBits);
        run += valid ? seq_items(a, lens[s]) : 0;
      } else {
        prefix[j] = run;
        run += seq_items(a, lens[j]);
      }
    }
  }
  if (tid == 255) prefix[S] = run;  // thread 255 holds the grand total (its chunk ends at S or later)
  __syncthreads();

  // Prefix groups: list order (chunk, 64-row group, KV head) with the KV head fastest.
  const int G = gridDim.x;
  constexpr int kGroupRows = 16 * kPrefixTiles * kWaves;
  const int n_groups = kPre && a.prefix_len > 0 ? (S * g + kGroupRows - 1) / kGroupRows : 0;
  const int n_pre = n_groups * a.prefix_chunks * H;
  if constexpr (kPre) {
    for (int i = blockIdx.x; i < n_pre; i += G) {
      const int h = i % H, t = (i / H) % n_groups, c = i / (H * n_groups);
      const int start = c * kPrefixChunk;
      const int end = min(a.prefix_len, start + kPrefixChunk);
      prefix_group<CT, QT, D>(a, lens, h, kGroupRows * t + 16 * kPrefixTiles * w, start / kBlock,
                              end / kBlock, end, c,
                              first_table_entries(a.prefix_table, start / kBlock, end / kBlock));
    }
  }
  // The sequences' items, one per wavefront.  Wavefronts are ranked so that those of workgroups
  // without prefix work come first, each class wavefront-major (wavefront w of every workgroup
  // before wavefront w + 1 of any): the first items go one to every workgroup, spread over all
  // compute units, before any workgroup gets a second.  Item f goes to the wavefront of rank
  // f mod 4G.  The list is (sequence, partition, KV head) with the KV head fastest, so the
  // wavefronts running at the same time cover the H tiles (b, 0..H-1) of the same blocks, next to
  // each other in the pool.
  const int busy = min(n_pre, G);  // workgroups 0 .. busy - 1 have prefix work
  // Workgroup b runs on compute unit b mod N (N = num_cus) when the grid is a whole number of
  // workgroups per unit.  With prefix work on units 0 .. busy - 1 only, the other units would hold
  // one more item workgroup each; that last one (b >= G - N + busy) is ranked after all other item
  // workgroups, so the wavefronts left without an item are there, and every unit streams about the
  // same number of items.
  const int N = a.num_cus;
  const bool spread = kPre && busy > 0 && N > 0 && busy < N && G % N == 0 && G >= 2 * N;
  const int nA = spread ? G - N : G - busy;  // item workgroups ranked first
  const int cb = G - N + busy;               // first of the late item workgroups (spread)
  const int b = blockIdx.x;
  const int rank = b < busy ? (G - busy) * kWaves + w * busy + b
                   : (!spread || b < cb) ? w * nA + (b - busy)
                                         : nA * kWaves + w * (N - busy) + (b - cb);
  const int total = __builtin_amdgcn_readfirstlane(prefix[S]) * H;
  const int GW = G * kWaves;
  auto item_of = [&](int f) {
    const int pf = f / H;
    const int h = f - pf * H;
    const int cmask = ord ? (1 << kOrderCountBits) - 1 : -1;
    int lo = 0, hi = S - 1;  // largest entry whose count is <= pf (LDS values, made uniform)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((__builtin_amdgcn_readfirstlane(prefix[mid]) & cmask) <= pf) lo = mid;
      else hi = mid - 1;
    }
    const int e = __builtin_amdgcn_readfirstlane(prefix[lo]);
    const int s = ord ? (int)((unsigned)e >> kOrderCountBits) : lo;
    return sequence_item(a, s, __builtin_amdgcn_readfirstlane(lens[s]), pf - (e & cmask), h);
  };
  // The next item's coordinates and first table entries are fetched before the current item
  // streams, so an item starts with one round trip to memory (its first blocks, with its query)
  // instead of three (context length, table, blocks).
  if (rank < total) {
    SeqItem it = item_of(rank);
    int tbl = item_table_entries<kB>(a, it);
    asm volatile("" : "+v"(tbl));  // waited for here, once, not at the loop header every item
    for (int f = rank; f < total; f += GW) {
      SeqItem next = it;
      int tbl_next = -1;
      if (f + GW < total) {
        next = item_of(f + GW);
        tbl_next = item_table_entries<kB>(a, next);
      }
      run_sequence_item<CT, QT, D, kB, kApp, kPair>(a, it, tbl, tbl_next);
      it = next;
      tbl = tbl_next;
    }
  }
  if constexpr (kApp) write_token_rows<CT, QT, D>(a, rank, GW);
}

// ---------------------------------------------------------------------------------------------

// Compute units of the current device, looked up once per device.
int device_cus() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  const int c = cache[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return 0;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Whether a plain decode takes its partitions two to a wavefront item (pair_items).  One wavefront
// streaming a row's blocks in one long run outpaces two wavefronts of a SIMD streaming them as two
// items, and the boundary between the two partitions costs the ring nothing.  Pairs are taken where
// the list at one partition per item holds between one and two items per SIMD: one round either
// way, and the pairs still give every SIMD a wavefront.  The count takes every row at the call's
// largest partition count (the host does not see the context lengths).
bool pair_items(const DecodeArgs &a) {
  if (a.prefix_len > 0 || a.cache.block_size != kBlock ||
      a.num_seqs > kMaxScanSeqs || a.num_partitions < 2)
    return false;
  const int cus = device_cus();
  if (cus <= 0) return false;
  const int64_t simds = (int64_t)cus * 4;
  const int64_t items = (int64_t)a.num_seqs * a.cache.num_kv_heads * a.num_partitions;
  return items > simds && items <= 2 * simds;
}

template <class CT, class QT, int D, bool kPre, int kB, bool kApp, bool kPair>
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
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &occ, decode_mfma_kernel<CT, QT, D, kPre, kB, kApp, kPair>, 256, 0) !=
          hipSuccess || occ < 1)
    occ = 1;
  if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                     hipSuccess || cus < 1)
    cus = 1;
  const int n = occ * cus;
  if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// The instantiation a call runs on, as a tag type for with_kernel's visitor.
template <class CT_, class QT_, int D_, bool kPre_, int kB_, bool kApp_, bool kPair_ = false>
struct KernelCfg {
  using CT = CT_;
  using QT = QT_;
  static constexpr int D = D_, kB = kB_;
  static constexpr bool kPre = kPre_, kApp = kApp_, kPair = kPair_;
};

// Calls f(KernelCfg<...>{}) for the instantiation that computes `a`: cache dtype, head_dim, shared
// prefix, block size, and the fused append (an instantiation of its own, so that the plain decode
// keeps its registers).
template <class CT, class QT, int D, bool kPre, int kB, class F>
auto with_app(const DecodeArgs &a, F &&f) {
  if constexpr (!kPre && kB == 16)
    if (a.pair_items)
      return a.append_slots ? f(KernelCfg<CT, QT, D, false, 16, true, true>{})
                            : f(KernelCfg<CT, QT, D, false, 16, false, true>{});
  return a.append_slots ? f(KernelCfg<CT, QT, D, kPre, kB, true>{})
                        : f(KernelCfg<CT, QT, D, kPre, kB, false>{});
}

template <class CT, class QT, int D, class F>
auto with_blocks(const DecodeArgs &a, F &&f) {
  if (a.prefix_len > 0) return with_app<CT, QT, D, true, 16>(a, f);
  switch (a.cache.block_size) {
    case 8: return with_app<CT, QT, D, false, 8>(a, f);
    case 32: return with_app<CT, QT, D, false, 32>(a, f);
    default: return with_app<CT, QT, D, false, 16>(a, f);
  }
}

template <class CT, class QT, class F>
auto with_dim(const DecodeArgs &a, F &&f) {
  return a.cache.head_dim == 64 ? with_blocks<CT, QT, 64>(a, f) : with_blocks<CT, QT, 128>(a, f);
}

// Grid of a call on the current device: direct (one wavefront per item, rounded up to whole
// workgroups) or persistent (every workgroup that fits at once, at most the direct count).
template <class C>
dim3 decode_grid(DecodeArgs &a) {
  const int64_t parts = C::kPair ? (a.num_partitions + 1) / 2 : a.num_partitions;
  const int64_t items = parts * a.cache.num_kv_heads * a.num_seqs;
  const int64_t direct = (items + kWaves - 1) / kWaves;
  a.persistent = a.num_seqs <= (C::kPre ? kMaxScanSeqsPrefix : kMaxScanSeqs);
  if (!a.persistent) return dim3((unsigned)direct);
  const int resident = resident_groups<typename C::CT, typename C::QT, C::D, C::kPre, C::kB,
                                       C::kApp, C::kPair>();
  return dim3((unsigned)std::min<int64_t>(direct, resident));
}

template <class C>
hipError_t launch_cfg(DecodeArgs a, hipStream_t s) {
  const dim3 grid = decode_grid<C>(a);
  a.num_cus = device_cus();
  decode_mfma_kernel<typename C::CT, typename C::QT, C::D, C::kPre, C::kB, C::kApp, C::kPair>
      <<<grid, dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// Wavefronts of the persistent grid that take sequence items (those of workgroups without prefix
// groups); 0 for the direct grid.
template <class C>
int item_waves_cfg(DecodeArgs a) {
  const int G = (int)decode_grid<C>(a).x;
  if (!a.persistent) return 0;
  int busy = 0;
  if (C::kPre && a.prefix_len > 0) {
    constexpr int kGroupRows = 16 * kPrefixTiles * kWaves;
    const int64_t n_groups = ((int64_t)a.num_seqs * (a.num_q_heads / a.cache.num_kv_heads) +
                              kGroupRows - 1) / kGroupRows;
    busy = (int)std::min<int64_t>(n_groups * a.prefix_chunks * a.cache.num_kv_heads, G);
  }
  return (G - busy) * kWaves;
}

template <class F>
auto with_kernel(const DecodeArgs &a, F &&f) {
  switch (a.cache.dtype) {
    case kBF16: return with_dim<bf16_t, bf16_t>(a, f);
    case kFP8: return with_dim<fp8_t, f16_t>(a, f);
    default: return with_dim<f16_t, f16_t>(a, f);
  }
}

}  // namespace

bool decode_mfma_supports_prefix(const DecodeArgs &a) {
  // the prefix groups exist only in the persistent grid
  return decode_mfma_supports(a) && a.num_seqs <= kMaxScanSeqsPrefix;
}

bool decode_mfma_supports(const DecodeArgs &a) {
  const int cdt = a.cache.dtype, qdt = a.q_dtype;
  const bool types = (cdt == kF16 && qdt == kF16) || (cdt == kBF16 && qdt == kBF16) ||
                     (cdt == kFP8 && qdt == kF16);
  const int g = a.num_q_heads / a.cache.num_kv_heads;
  // the Q^T operand is read as 16-byte vectors of 8 elements; outputs are stored 4 at a time
  const bool q_aligned = (reinterpret_cast<uintptr_t>(a.q) & 15u) == 0 && a.q_stride % 8 == 0 &&
                         (reinterpret_cast<uintptr_t>(a.out) & 7u) == 0;
  // an empty pool has no tile for the ring's idle slots to read
  return types && g >= 1 && g <= 16 && (a.cache.head_dim == 64 || a.cache.head_dim == 128) &&
         q_aligned && a.cache.num_blocks > 0;
}

hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
  if (a.cache.dtype != kF16 && a.cache.dtype != kBF16 && a.cache.dtype != kFP8)
    return hipErrorInvalidValue;
  DecodeArgs b = a;
  b.pair_items = pair_items(a) ? 1 : 0;
  return with_kernel(b, [&](auto c) { return launch_cfg<decltype(c)>(b, s); });
}

int decode_mfma_item_waves(const DecodeArgs &a) {
  if (a.cache.dtype != kF16 && a.cache.dtype != kBF16 && a.cache.dtype != kFP8) return 0;
  return with_kernel(a, [&](auto c) { return item_waves_cfg<decltype(c)>(a); });
}

}  // namespace pa
