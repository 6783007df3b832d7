// prefill_mfma.hip — paged prefill on the matrix cores of gfx950: a chunk of new tokens per
// sequence, each attending causally through the block table to its sequence's earlier positions
// and to the chunk's tokens before it ("PagedAttention, Visualized", Parts 1 and 2: a prompt passes
// through the model as one matrix whose tokens look at each other; a token's K and V serve every
// later token).  The chunk's K and V are already in the cache.
//
// This translation unit is compiled with -fno-honor-nans -mno-amdgpu-ieee (build.py): with the
// hardware's IEEE mode off, a maximum of two floats is one instruction, where IEEE mode makes the
// compiler quiet each operand first (one more instruction per score in the softmax).  No value
// here is tested for NaN: positions past a row's limit are excluded by selects on their index and
// V elements by bit masks, so NaN in the pool (the parity tests fill unused bytes with it) still
// cannot reach an output.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "mfma_common.h"
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

// Prefill (a chunk of n new tokens per sequence, positions L - n .. L - 1; the token at position p
// attends to positions 0 .. p).  Unlike decode, every block serves many rows, so the work is
// matrix-core bound, not memory bound, and is arranged for the products:
//  - workgroup (s, h, group) takes kPrefillRows rows of sequence s and KV head h (row r is token
//    r / g, query head h*g + r % g), its wavefront w kPrefillTiles tiles of 16 rows;
//  - the blocks go through LDS two at a time (a pair A, B: 32 positions), copied straight from the
//    pool (wavefront w copies tile w of the pair: K or V of block A or B) and read back by each
//    wavefront, so a block is fetched once per 128 rows;
//  - P V is one 16x16x32 product per 16 head dims over the pair, reduction index k = position
//    tok0 + k of the pair: lane group grp (lanes 16 grp ..) holds positions 8 grp .. 8 grp + 7,
//    i.e. 8 consecutive positions of block grp / 2, so its V^T operand is one 16-byte row piece;
//  - the scores come from two 16x16x32 products per pair, X on positions 8 q + 0..3 of each
//    block (q = 0, 1) and Y on 8 q + 4..7, whose result layouts put exactly those 8 positions in
//    lane group grp (X gives the first four, Y the next four);
//  - the LDS copy of a block is permuted so that every read of a product operand is a 16-byte
//    load free of bank conflicts: K vectors of a token row are swizzled (token bit 2 flips with
//    bit 3, block B also flips bit 3), 16-bit V^T tiles are stored half-row-major;
//  - the scores of a pair are taken together (one maximum update per pair, the row maximum by
//    lane swaps rather than LDS shuffles);
//  - probabilities are rounded once to the input type (no hi + lo split): each output averages
//    many positions, so the rounding of single probabilities does not accumulate;
//  - step k of a round computes pair k's softmax and P V and, beside that softmax, the score
//    products of pair k + 1, so the matrix pipe has work while the vector ALUs do the softmax.
// Each row masks the positions past its own; the workgroup walks the blocks up to its last row's
// position, in rounds of 64 blocks (one table fetch per round).  Rows are complete in one
// wavefront: the outputs are written directly, no workspace.
// Two 16-row tiles per wavefront, four pair stages in LDS, two wavefronts per SIMD (one tile at
// three per SIMD, and three, five or six stages, measured slower).
constexpr int kPrefillTiles = 2;
constexpr int kPrefillStages = 4;
constexpr int kPrefillOcc = 2;
constexpr int kXcds = 8;  // accelerator complex dies; workgroups are dealt to them round-robin
constexpr int kPrefillRows = 16 * kPrefillTiles * kWaves;

template <class CT, int D>
struct PairStages {
  static constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  static constexpr int kTileBytes = kBlock * D * CT::bytes;
  static constexpr int kBlockBytes = 2 * kTileBytes;  // K tile, then V tile
  static constexpr int kBytes = 2 * kBlockBytes;      // block A, then block B
  static constexpr int kChunks = kBytes / 1024;       // 1 KiB copies per pair
  static constexpr int kPerWave = kChunks / kWaves;
  static constexpr int kStages = kPrefillStages;
  static_assert(kChunks % kWaves == 0, "pair split");
};

// Token order of a K vector row in LDS: slot k_slot(t, b) (in 16-byte units, within its 16-slot
// row) holds token t of block b (0: A, 1: B); k_token is its inverse.
__device__ __forceinline__ int tok_swap(int t) { return t ^ (((t >> 3) & 1) << 2); }  // involution
__device__ __forceinline__ int k_slot(int t, int b) { return tok_swap(t) ^ (b << 3); }
__device__ __forceinline__ int k_token(int slot, int b) { return tok_swap(slot ^ (b << 3)); }

// Wavefront w copies tile w of every pair: the K tile (w = 0) or V tile (w = 1) of block A, or
// those of block B (w = 2, 3), in 1 KiB pieces j = 0 .. kTileBytes / 1024 - 1, permuted as the
// reads expect: LDS slot s of a K tile holds the pool's vector (s / 16, token k_token(s % 16));
// LDS slot s of a 16-bit V^T tile holds head dim s % D, positions 8 (s / D) .. + 7; fp8 V^T
// tiles are copied as they are.  Piece j's source offset is a per-lane part that does not depend
// on j (`voff`) plus a wave-uniform part (`piece_soff`), both fixed for the whole call.
struct PairCopy {
  const char *base;  // pool of this wavefront's tile, advanced to KV head h
  size_t stride;     // bytes between blocks in that pool (num_kv_heads tiles)
  int voff;          // per-lane source byte offset of every piece
  int blk;           // block of the pair this wavefront copies (0: A, 1: B)
  bool is_v;
};

template <class CT, int D>
__device__ __forceinline__ PairCopy pair_copy_setup(const DecodeArgs &a, int h) {
  using P = PairStages<CT, D>;
  const int lane = thread_x() & 63;
  const int w = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  PairCopy c;
  c.blk = w >> 1;
  c.is_v = (w & 1) != 0;
  c.stride = (size_t)a.cache.num_kv_heads * P::kTileBytes;
  c.base = static_cast<const char *>(c.is_v ? a.cache.v_pool : a.cache.k_pool) +
           (size_t)h * P::kTileBytes;
  if (!c.is_v) c.voff = 16 * ((lane & ~15) | k_token(lane & 15, c.blk));
  else c.voff = P::kFP8 ? 16 * lane : 32 * lane;
  return c;
}

// Wave-uniform source offset of piece j (LDS slots 64 j .. 64 j + 63 of the tile).
template <class CT, int D>
__device__ __forceinline__ int piece_soff(const PairCopy &c, int j) {
  using P = PairStages<CT, D>;
  if (P::kFP8 || !c.is_v) return 1024 * j;
  return 16 * (2 * ((64 * j) % D) + (64 * j) / D);  // slot 64 j + lane -> 2 (slot % D) + slot / D
}

// This wavefront's tile of the pair (blocks ba, bb of KV head h) into stage I; an absent block
// copies through an empty descriptor and touches no memory.
template <class CT, int D, int I>
__device__ __forceinline__ void stage_pair(const PairCopy &c, int ba, bool oka, int bb, bool okb) {
  using P = PairStages<CT, D>;
  constexpr int kPieces = P::kTileBytes / 1024;
  static_assert(kPieces * kWaves == P::kChunks, "one tile per wavefront");
  const int b = c.blk ? bb : ba;
  const bool ok = c.blk ? okb : oka;
  const auto r = tile_rsrc(c.base + (size_t)(ok ? b : 0) * c.stride, ok ? P::kTileBytes : 0);
  auto *dst = prefix_stage<P::kBytes, 16 + I>() + (2 * c.blk + (c.is_v ? 1 : 0)) * P::kTileBytes;
#pragma unroll
  for (int j = 0; j < kPieces; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (PA_LDS void *)(dst + 1024 * j), 16, c.voff,
                                             piece_soff<CT, D>(c, j), 0, 0);
}

// K operand of score product X (which = 0) or Y (which = 1), vector i (16 dims of fp8, 8 of
// 16-bit): lane (r = lane / 16, c = lane % 16) holds vector 4 i + r of position
// 8 ((c >> 2) & 1) + 4 which + (c & 3) of block c >> 3.
template <class CT, int D, int I, int kWhich, int N>
__device__ __forceinline__ void read_pair_k(uint4 (&k)[N]) {
  using P = PairStages<CT, D>;
  const int lane = thread_x() & 63, c = lane & 15, r = lane >> 4;
  const int b = c >> 3;
  const int t = 8 * ((c >> 2) & 1) + 4 * kWhich + (c & 3);
  const auto *base = prefix_stage<P::kBytes, 16 + I>() + b * P::kBlockBytes +
                     (16 * r + k_slot(t, b)) * 16;
#pragma unroll
  for (int i = 0; i < N; ++i) k[i] = lds_load<uint4>(base + 64 * 16 * i);
}

// V^T operand for head dims 16 nt + c (c = lane % 16) and positions 8 grp .. 8 grp + 7 of the pair
// (grp = lane / 16: block grp / 2, its positions 8 (grp % 2) ..), as 8 values of the product type.
template <class CT, int D, int I>
__device__ __forceinline__ uint4 read_pair_v(int nt) {
  using P = PairStages<CT, D>;
  const int lane = thread_x() & 63, c = lane & 15, grp = lane >> 4;
  const auto *tile = prefix_stage<P::kBytes, 16 + I>() + (grp >> 1) * P::kBlockBytes + P::kTileBytes;
  if constexpr (P::kFP8) {
    const uint2 x = lds_load<uint2>(tile + (16 * nt + c) * kBlock + 8 * (grp & 1));
    const uint2 lo = e4m3x4_to_f16x4(x.x), hi = e4m3x4_to_f16x4(x.y);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    return lds_load<uint4>(tile + ((grp & 1) * D + 16 * nt + c) * 16);
  }
}

// S^T of one score product against this wavefront tile's query rows (raw products).
template <class CT, int D, int N>
__device__ __forceinline__ f4_t block_qk(const uint4 (&k)[N], const RowState<D> &rs_) {
  constexpr bool kFP8 = std::is_same<CT, fp8_t>::value;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;
  f4_t st = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (kFP8) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const uint2 a0 = e4m3x4_to_f16x4(k[i].x), a1 = e4m3x4_to_f16x4(k[i].y);
      const uint2 a2 = e4m3x4_to_f16x4(k[i].z), a3 = e4m3x4_to_f16x4(k[i].w);
      st = mma_k32<false>(make_uint4(a0.x, a0.y, a1.x, a1.y), rs_.qop[2 * i], st);
      st = mma_k32<false>(make_uint4(a2.x, a2.y, a3.x, a3.y), rs_.qop[2 * i + 1], st);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < N; ++kk) st = mma_k32<kBF>(k[kk], rs_.qop[kk], st);
  }
  return st;
}

// Maxima over the four 16-lane rows of a wavefront (lanes c, c + 16, c + 32, c + 48) of two values
// at once, t and u (the two tiles' pair maxima), by three lane swaps on the vector ALU: the first
// swap pairs row 1 of t with row 0 of u (and row 3 with row 2), so one maximum leaves t's rows
// {0, 1} and {2, 3} reduced in rows 0 and 2 and u's in rows 1 and 3; swapping the halves reduces
// over all four rows; a last swap of rows hands every lane both results.
__device__ __forceinline__ void max_over_rows2(float &t, float &u) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(u), false,
                                                  false);
  const float m1 = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(m1), false,
                                                  false);
  const float m2 = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(m2), __float_as_uint(m2), false,
                                                  false);
  t = __uint_as_float(c[0]);
  u = __uint_as_float(c[1]);
}

// Softmax over a pair, in two parts, so that the next pair's score products can be issued beside
// each.  z holds this lane's raw scores of the pair, positions 8 grp + i, i < 8 (product X gives
// i < 4, product Y the rest); ks > 0 is the logit scale (a negative scale is folded into the
// query's sign, a zero one replaced by the smallest normal float, which leaves every probability
// at exactly 1 as a zero scale does).
// Part 1: the pair's row maxima of both tiles, scaled once; grow[j] says whether tile j's exceeds
// its running maximum by more than kSlack (base 2), when its running state must be rescaled.
template <int D>
__device__ __forceinline__ void pair_max2(const float (&z)[2][8], float ks, const RowState<D> (&rs)[2],
                                          float (&mx)[2], bool (&grow)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    mx[j] = fmaxf(fmaxf(fmaxf(z[j][0], z[j][1]), fmaxf(z[j][2], z[j][3])),
                  fmaxf(fmaxf(z[j][4], z[j][5]), fmaxf(z[j][6], z[j][7])));
  max_over_rows2(mx[0], mx[1]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    mx[j] *= ks;  // -inf stays -inf
    grow[j] = mx[j] > rs[j].m + kSlack;
  }
}

// Rescale this lane's running state to the new maximum mx when `grow` (per lane).
template <int D>
__device__ __forceinline__ void pair_rescale(bool grow, float mx, RowState<D> &rs_) {
  const float mn = grow ? mx : rs_.m;
  const float alpha = __builtin_amdgcn_exp2f(rs_.m - mn);
  rs_.l *= alpha;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) rs_.acc[nt] *= alpha;
  rs_.m = mn;
}

// Part 2: each probability 2^(s * ks - m) in one fused multiply-add, their sum added to l; returns
// this lane's P^T operand, the 8 probabilities in position order rounded to the input type.
template <class CT, int D>
__device__ __forceinline__ uint4 pair_probs(const float (&z)[8], float ks, RowState<D> &rs_) {
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[i], ks, -rs_.m));
  rs_.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  return make_uint4(pack2_pk<kBF>(p[0], p[1]), pack2_pk<kBF>(p[2], p[3]),
                    pack2_pk<kBF>(p[4], p[5]), pack2_pk<kBF>(p[6], p[7]));
}

// Mask words that zero the 16-bit V values of this lane's positions 8 grp + i of the pair at or
// past rel (this lane's limit minus 8 grp), two positions per word.
__device__ __forceinline__ uint4 pair_keep(int rel) {
  auto two = [&](int i) { return (i < rel ? 0xffffu : 0u) | (i + 1 < rel ? 0xffff0000u : 0u); };
  return make_uint4(two(0), two(2), two(4), two(6));
}

template <class CT, class QT, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kPrefillOcc)))
void prefill_mfma_kernel(DecodeArgs a) {
  using P = PairStages<CT, D>;
  using F = Frag<CT, D>;
  constexpr int kS = P::kStages;
  constexpr int kT = kPrefillTiles;
  constexpr bool kBF = std::is_same<CT, bf16_t>::value;
  const int w = __builtin_amdgcn_readfirstlane(thread_x() >> 6);
  const int H = a.cache.num_kv_heads, g = a.num_q_heads / H;
  const int groups = (a.max_query_len * g + kPrefillRows - 1) / kPrefillRows;
  // Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD takes a contiguous range of the
  // list (sequence, KV head, group), so the groups that re-read one sequence's blocks share an L2.
  // Within a (sequence, KV head) the longest groups (the last rows of a prompt attend to the most
  // positions) come first.
  const int per_xcd = (int)(grid_x() / kXcds);
  const int f = (int)(block_x() % kXcds) * per_xcd + (int)(block_x() / kXcds);
  if (f >= a.num_seqs * H * groups) return;  // the grid's padding to a multiple of kXcds
  const int gi = groups - 1 - f % groups;
  const int sh = f / groups;
  const int h = sh % H, s = sh / H;
  const int qs = a.query_start[s];
  const int n = min(a.query_start[s + 1] - qs, a.max_query_len);
  const int L = clamp_len(a, s);
  const int nrows = n * g;
  const int rbase = kPrefillRows * gi;
  if (n <= 0 || rbase >= nrows) return;  // workgroup-uniform, before any barrier
  const int last = min(rbase + kPrefillRows - 1, nrows - 1);
  const int end = max(0, min(L, L - n + last / g + 1));  // the workgroup's last row's limit
  const int col = thread_x() & 15;
  const int grp = (thread_x() & 63) >> 4;
  RowState<D> st[kT];
  bool rvalid[kT];
  int rs[kT], rhq[kT], lim[kT];
#pragma unroll
  for (int j = 0; j < kT; ++j) {
    const int r = rbase + 16 * (kT * w + j) + col;
    rvalid[j] = r < nrows;
    const int t = rvalid[j] ? r / g : 0;
    rs[j] = qs + t;
    rhq[j] = h * g + (rvalid[j] ? r % g : 0);
    lim[j] = max(0, min(L, L - n + t + 1));
    load_query<CT, D>(a, rs[j], rhq[j], rvalid[j], st[j]);
  }
  float kscale, vscale;
  head_scales<CT>(a, h, kscale, vscale);
  // The logit scale enters as ks > 0: a negative scale flips the sign of the query operand (the
  // products then come out exactly negated), a zero scale becomes the smallest normal float.
  const float ks = fabsf(kscale) == 0.0f ? 1.17549435e-38f : fabsf(kscale);
  if (kscale < 0.0f) {
#pragma unroll
    for (int j = 0; j < kT; ++j)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        st[j].qop[kk].x ^= 0x80008000u;
        st[j].qop[kk].y ^= 0x80008000u;
        st[j].qop[kk].z ^= 0x80008000u;
        st[j].qop[kk].w ^= 0x80008000u;
      }
  }
  // the smallest limit of this wavefront's rows (wave-uniform): pairs below it need no score mask
  int lmin = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kT; ++j) lmin = min(lmin, rvalid[j] ? lim[j] : 0x7fffffff);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lmin = min(lmin, __shfl_xor(lmin, o));
  lmin = __builtin_amdgcn_readfirstlane(lmin);
  const int32_t *table = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int nb = a.cache.num_blocks;
  const int jb1 = (end + kBlock - 1) / kBlock;
  const PairCopy pc = pair_copy_setup<CT, D>(a, h);
  int tbl = first_table_entries(table, 0, jb1);
#pragma unroll
  for (int j = 0; j < kT; ++j)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      asm volatile("" : "+v"(st[j].qop[kk].x), "+v"(st[j].qop[kk].y), "+v"(st[j].qop[kk].z),
                   "+v"(st[j].qop[kk].w));
  // The pairs of a round go through the stages in order; step k computes the softmax and P V of
  // pair k and, beside that softmax, the score products of pair k + 1 (its K tiles are in LDS by
  // then), so the matrix cores have work while the vector ALUs do the softmax.
  for (int c0 = 0; c0 < jb1; c0 += 64) {  // rounds of up to 64 blocks
    const int nk = min(64, jb1 - c0);
    const int npair = (nk + 1) / 2;
    // the next round's entries, waited for at its start
    int tbl_next = c0 + 64 < jb1 ? first_table_entries(table, c0 + 64, jb1) : -1;
    asm volatile("" : "+v"(tbl));
    auto id = [&](int b) { return b < nk ? __builtin_amdgcn_readlane(tbl, b) : -1; };
    int pid[kS][2];  // block ids of the pair in each stage, kept from its copy to its step
    auto issue = [&](auto I, int k) {  // pair k into stage I (past the end: empty copies)
      constexpr int i = decltype(I)::value;
      pid[i][0] = id(2 * k);
      pid[i][1] = id(2 * k + 1);
      stage_pair<CT, D, i>(pc, pid[i][0], (unsigned)pid[i][0] < (unsigned)nb, pid[i][1],
                           (unsigned)pid[i][1] < (unsigned)nb);
    };
    // Raw scores of the pair in stage I, this lane's 8 positions per tile (X then Y products).
    auto scores_x = [&](auto I, float (&z)[kT][8]) {
      uint4 kf[F::kKLoads];
      read_pair_k<CT, D, decltype(I)::value, 0>(kf);
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        const f4_t x = block_qk<CT, D>(kf, st[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[j][i] = x[i];
      }
    };
    auto scores_y = [&](auto I, float (&z)[kT][8]) {
      uint4 kf[F::kKLoads];
      read_pair_k<CT, D, decltype(I)::value, 1>(kf);
#pragma unroll
      for (int j = 0; j < kT; ++j) {
        const f4_t y = block_qk<CT, D>(kf, st[j]);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[j][4 + i] = y[i];
      }
    };
    float zc[kT][8];  // scores of the current pair
    auto step = [&](auto I, int k) {
      constexpr int i = decltype(I)::value;
      constexpr int inext = (i + 1) % kS;
      // pair k + 1 landed for every wavefront, and every wavefront is done with pair k - 1's stage
      stage_barrier<P::kPerWave * (kS - 3)>();
      issue(std::integral_constant<int, (i + kS - 1) % kS>{}, k + kS - 1);
      const bool oka = (unsigned)pid[i][0] < (unsigned)nb, okb = (unsigned)pid[i][1] < (unsigned)nb;
      // this lane's block is present (read only inside the masked branches)
      auto okm = [&]() { return (grp >> 1) ? okb : oka; };
      const int t0 = (c0 + 2 * k) * kBlock;
      const int tl = t0 + 8 * grp;  // this lane's first position of the pair
      // Masks only where they change something (wave-uniform tests): the scores where some row's
      // limit falls inside the pair, the V values where the pair reaches the workgroup's end
      // (positions past it may hold anything, NaN included); an absent block masks both.
      const bool both = oka && okb;
      const bool zmask = !both || t0 + 2 * kBlock > lmin;
      const bool vmask = !both || t0 + 2 * kBlock > end;
      if (zmask) {
#pragma unroll
        for (int j = 0; j < kT; ++j) {
          const int rel = (okm() ? lim[j] : 0) - tl;
#pragma unroll
          for (int q = 0; q < 8; ++q) zc[j][q] = q < rel ? zc[j][q] : -INFINITY;  // never NaN
        }
      }
      // Pair k + 1's X products beside pair k's maxima.  Past the round's last pair the stage
      // holds an empty copy (zeros); those scores are not used.
      float zn[kT][8];
      scores_x(std::integral_constant<int, inext>{}, zn);
      float mx[kT];
      bool grow[kT];
      static_assert(kT == 2, "the row maxima are reduced two tiles at a time");
      pair_max2<D>(zc, ks, st, mx, grow);
      if ((__builtin_amdgcn_ballot_w64(grow[0]) | __builtin_amdgcn_ballot_w64(grow[1])) != 0) {
#pragma unroll
        for (int j = 0; j < kT; ++j) pair_rescale(grow[j], mx[j], st[j]);
      }
      // Pair k + 1's Y products beside pair k's probabilities.
      scores_y(std::integral_constant<int, inext>{}, zn);
      uint4 pop[kT];
#pragma unroll
      for (int j = 0; j < kT; ++j) pop[j] = pair_probs<CT, D>(zc[j], ks, st[j]);
      if (!vmask) {
        // every V^T read issued before the products, so the LDS latency is paid once per pair
        uint4 vop[F::kNT];
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt) vop[nt] = read_pair_v<CT, D, i>(nt);
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt)
#pragma unroll
          for (int j = 0; j < kT; ++j) st[j].acc[nt] = mma_k32<kBF>(vop[nt], pop[j], st[j].acc[nt]);
        __builtin_amdgcn_sched_group_barrier(0x100, F::kNT, 0);       // the LDS reads first,
        __builtin_amdgcn_sched_group_barrier(0x8, F::kNT * kT, 0);    // then the products
      } else {
        const uint4 keep = pair_keep((okm() ? end : 0) - tl);
#pragma unroll
        for (int nt = 0; nt < F::kNT; ++nt) {
          uint4 vop = read_pair_v<CT, D, i>(nt);
          vop.x &= keep.x;  // a select: NaN in a masked position cannot leak
          vop.y &= keep.y;
          vop.z &= keep.z;
          vop.w &= keep.w;
#pragma unroll
          for (int j = 0; j < kT; ++j) st[j].acc[nt] = mma_k32<kBF>(vop, pop[j], st[j].acc[nt]);
        }
      }
#pragma unroll
      for (int j = 0; j < kT; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) zc[j][q] = zn[j][q];
    };
    stage_barrier<63>();  // the stages' previous readers are done
    static_for<0, kS - 1>([&](auto I) { issue(I, decltype(I)::value); });
    stage_barrier<P::kPerWave * (kS - 2)>();  // pair 0 landed for every wavefront
    scores_x(std::integral_constant<int, 0>{}, zc);
    scores_y(std::integral_constant<int, 0>{}, zc);
    int k0 = 0;
    for (; k0 + kS <= npair; k0 += kS)
      static_for<0, kS>([&](auto I) { step(I, k0 + decltype(I)::value); });
    static_for<0, kS>([&](auto I) {
      if (k0 + decltype(I)::value < npair) step(I, k0 + decltype(I)::value);
    });
    tbl = tbl_next;
  }
#pragma unroll
  for (int j = 0; j < kT; ++j)
    emit_rows<QT, D>(a, st[j], vscale, vscale, -1, rs[j], rhq[j], rvalid[j]);
}

template <class CT, class QT, int D>
hipError_t launch_prefill_dd(const DecodeArgs &a, hipStream_t s) {
  const int g = a.num_q_heads / a.cache.num_kv_heads;
  const int64_t groups = ((int64_t)a.max_query_len * g + kPrefillRows - 1) / kPrefillRows;
  const int64_t items = (int64_t)a.num_seqs * a.cache.num_kv_heads * groups;
  if (items == 0) return hipSuccess;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  prefill_mfma_kernel<CT, QT, D><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

template <class CT, class QT>
hipError_t launch_prefill_d(const DecodeArgs &a, hipStream_t s) {
  return a.cache.head_dim == 64 ? launch_prefill_dd<CT, QT, 64>(a, s)
                                : launch_prefill_dd<CT, QT, 128>(a, s);
}

}  // namespace

hipError_t launch_prefill_mfma(const DecodeArgs &a, hipStream_t s) {
  switch (a.cache.dtype) {
    case kF16: return launch_prefill_d<f16_t, f16_t>(a, s);
    case kBF16: return launch_prefill_d<bf16_t, bf16_t>(a, s);
    case kFP8: return launch_prefill_d<fp8_t, f16_t>(a, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace pa
