/*
 * oracle.c — TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct CPU reference for decode-step
 * paged attention, in fp64.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this file's library; the product never does.  It shares no code with the GPU path:
 * element decoders, the pool indexer, the fp8 codec and the attention are all written here again
 * from their definitions.
 *
 * Sources (web pages, cited by title and section):
 *   [Visualized] "PagedAttention, Visualized" — Part 2 (K and V are kept per token), Part 3 (blocks,
 *                block table, shared prefix blocks).
 *   [Digest]     "PagedAttention" (devoured.fyi) — "PagedAttention in one picture" (pool of 16-token
 *                blocks, block table logical -> physical, the kernel walks the table), "Copy-on-write:
 *                when two requests share a prefix" (clone, decrement, retarget), "Misconceptions"
 *                (attention math unchanged whether K/V are contiguous or scattered).
 *   [Lesson06]   "LLM Inference Visualizer, Lesson 06" — "How paging grows" (each token appends one
 *                KV entry in the current block).
 * The pool layout is the library's own, read from the prose in include/pa.h, not from its code.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py (none is "parity unpinned").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8 = 3 };

int orc_elem_bytes(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8: return 1;
    default: return 0;
  }
}

/* ---------------------------------------------------------------- element decoders (exact) ---- */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = h >> 15, ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
  double v;
  if (ex == 0) {
    v = ldexp((double)fr, -24); /* subnormal: fr * 2^-10 * 2^-14 */
  } else if (ex == 31) {
    v = fr ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + fr), ex - 25); /* (1 + fr/1024) * 2^(ex-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction bits; S.1111.111 is NaN, no infinities. */
double orc_e4m3_to_f64(uint8_t c) {
  int sign = c >> 7, ex = (c >> 3) & 0xF, fr = c & 0x7;
  double v;
  if (ex == 15 && fr == 7) return NAN;
  if (ex == 0) {
    v = ldexp((double)fr, -9); /* subnormal: fr/8 * 2^(1-7) */
  } else {
    v = ldexp((double)(8 + fr), ex - 10); /* (1 + fr/8) * 2^(ex-7) */
  }
  return sign ? -v : v;
}

/* Encode a binary32 value as E4M3FN: nearest representable value, ties to the even code (even
 * fraction), magnitudes at or above the largest finite value 448 saturate to 448, NaN -> 0x7F with
 * the sign bit of the input.  The 127 non-negative finite codes 0x00 .. 0x7E have values that
 * increase with the code, so the largest code whose value does not exceed |x| is found by bisection
 * over them (the decoder above gives each code's value). */
uint8_t orc_e4m3_from_f32(float x) {
  uint32_t bits;
  memcpy(&bits, &x, sizeof bits);
  uint8_t sign = (uint8_t)((bits >> 31) << 7);
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)x);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  /* largest code with value <= a: value(lo) <= a < value(hi) holds throughout (value(0) = 0) */
  int lo = 0, hi = 0x7F;
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (orc_e4m3_to_f64((uint8_t)mid) <= a) lo = mid;
    else hi = mid;
  }
  int code = lo;
  if (lo < 0x7E) {
    double vlo = orc_e4m3_to_f64((uint8_t)lo), vhi = orc_e4m3_to_f64((uint8_t)(lo + 1));
    double dlo = a - vlo, dhi = vhi - a;
    if (dhi < dlo || (dhi == dlo && (lo & 1))) code = lo + 1;
  }
  return (uint8_t)(sign | code);
}

/* Exact value of element `idx` of an array of `dtype` elements. */
static double load_elem(const void *base, int dtype, size_t idx) {
  switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_F16: return orc_f16_to_f64(((const uint16_t *)base)[idx]);
    case ORC_BF16: return orc_bf16_to_f64(((const uint16_t *)base)[idx]);
    case ORC_FP8: return orc_e4m3_to_f64(((const uint8_t *)base)[idx]);
    default: abort();
  }
}

/* Exact binary32 value of an f32/f16/bf16 element (all three embed exactly in binary32). */
static float load_elem_f32(const void *base, int dtype, size_t idx) {
  return (float)load_elem(base, dtype, idx);
}

/* ------------------------------------------------------------------- pool indexer ------------- */
/* Element index, within one pool, of (block b, kv head h, token slot t, head-dim index i), as
 * include/pa.h describes the layout: tile (b, h) starts at (b*H + h)*B*D; in a K tile element
 * (t, i) is at ((i / E)*B + t)*E + i % E with E = 16 / element bytes; in a V tile at i*B + t. */
size_t orc_k_index(int b, int h, int t, int i, int H, int D, int B, int dtype) {
  size_t E = (size_t)(16 / orc_elem_bytes(dtype));
  size_t tile = ((size_t)b * H + h) * (size_t)B * D;
  return tile + ((size_t)(i / E) * B + t) * E + (size_t)(i % E);
}

size_t orc_v_index(int b, int h, int t, int i, int H, int D, int B) {
  size_t tile = ((size_t)b * H + h) * (size_t)B * D;
  return tile + (size_t)i * B + t;
}

/* ------------------------------------------------------------------- de-paging ---------------- */
/* Gather the first L positions of one sequence's KV head h into contiguous fp64 arrays
 * kc[L][D], vc[L][D]: position p lives in physical block table[p / B] at slot p % B ([Digest]
 * "PagedAttention in one picture").  fp8 elements are multiplied by their head's scale (exact in
 * fp64).  Returns -1 (and reads nothing further) if a referenced block id is out of range. */
int orc_gather(double *kc, double *vc, const void *k_pool, const void *v_pool, int cache_dtype,
               const float *k_scale, const float *v_scale, int num_blocks, int H, int D, int B,
               const int32_t *table, int L, int h) {
  for (int p = 0; p < L; ++p) {
    int b = table[p / B];
    if (b < 0 || b >= num_blocks) return -1;
    int t = p % B;
    for (int i = 0; i < D; ++i) {
      double kv = load_elem(k_pool, cache_dtype, orc_k_index(b, h, t, i, H, D, B, cache_dtype));
      double vv = load_elem(v_pool, cache_dtype, orc_v_index(b, h, t, i, H, D, B));
      if (cache_dtype == ORC_FP8) {
        kv *= (double)k_scale[h];
        vv *= (double)v_scale[h];
      }
      kc[(size_t)p * D + i] = kv;
      vc[(size_t)p * D + i] = vv;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------- attention ---------------- */
/* Ordinary attention of one query row over contiguous K/V: z_p = scale * <q, k_p>,
 * out = sum_p exp(z_p - max z) v_p / sum_p exp(z_p - max z); out = 0 when L == 0. */
static void attend(double *out, const double *q, const double *kc, const double *vc, int L, int D,
                   double scale) {
  for (int i = 0; i < D; ++i) out[i] = 0.0;
  if (L == 0) return;
  double *z = (double *)malloc(sizeof(double) * (size_t)L);
  double m = -INFINITY;
  for (int p = 0; p < L; ++p) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += q[i] * kc[(size_t)p * D + i];
    z[p] = scale * acc;
    if (z[p] > m) m = z[p];
  }
  double den = 0.0;
  for (int p = 0; p < L; ++p) {
    double w = exp(z[p] - m);
    den += w;
    for (int i = 0; i < D; ++i) out[i] += w * vc[(size_t)p * D + i];
  }
  for (int i = 0; i < D; ++i) out[i] /= den;
  free(z);
}

/*
 * Decode attention for the (sequence, query head) pairs sel_seq[k], sel_head[k], k < nsel
 * (nsel < 0: every pair, in order s-major).  out is [nsel][D] fp64 (or [S][Hq][D] for all pairs).
 * Each pair: de-page the sequence's KV head h = q_head / (Hq / H), then attend.  q is [S] rows of
 * Hq*D elements of q_dtype, q_stride elements apart.  Returns 0, or -1 if a referenced block id is
 * out of range, -2 on bad sizes.
 */
int orc_decode_attention(double *out, const void *q, int q_dtype, int64_t q_stride,
                         const void *k_pool, const void *v_pool, int cache_dtype,
                         const float *k_scale, const float *v_scale, int num_blocks, int H, int D,
                         int B, const int32_t *block_tables, int max_blocks_per_seq,
                         const int32_t *context_lens, int S, int Hq, float scale,
                         const int32_t *sel_seq, const int32_t *sel_head, int nsel, int nthreads) {
  if (H <= 0 || Hq % H != 0 || D <= 0 || B <= 0) return -2;
  int g = Hq / H;
  if (q_stride == 0) q_stride = (int64_t)Hq * D;
  long total = nsel < 0 ? (long)S * Hq : nsel;
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
  for (long k = 0; k < total; ++k) {
    int s = nsel < 0 ? (int)(k / Hq) : sel_seq[k];
    int hq = nsel < 0 ? (int)(k % Hq) : sel_head[k];
    int L = context_lens[s];
    if (L < 0 || L > max_blocks_per_seq * B) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = -2;
      continue;
    }
    int h = hq / g;
    double *qd = (double *)malloc(sizeof(double) * (size_t)D);
    double *kc = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
    double *vc = (double *)malloc(sizeof(double) * ((size_t)L * D + 1));
    for (int i = 0; i < D; ++i)
      qd[i] = load_elem(q, q_dtype, (size_t)s * q_stride + (size_t)hq * D + i);
    const int32_t *table = block_tables + (size_t)s * max_blocks_per_seq;
    if (orc_gather(kc, vc, k_pool, v_pool, cache_dtype, k_scale, v_scale, num_blocks, H, D, B,
                   table, L, h) != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = -1;
    } else {
      attend(out + (size_t)k * D, qd, kc, vc, L, D, (double)scale);
    }
    free(qd);
    free(kc);
    free(vc);
  }
  return status;
}

/* Ordinary attention on caller-provided contiguous fp64 K/V (kc, vc: [L][D]); exposed so tests can
 * check the de-paging step separately from the softmax step. */
void orc_attend_contiguous(double *out, const double *q, const double *kc, const double *vc, int L,
                           int D, double scale) {
  attend(out, q, kc, vc, L, D, scale);
}

/* ------------------------------------------------------------ reshape_and_cache replay -------- */
/* For each token t with slot s = slots[t] in [0, num_blocks*B): write K row t and V row t (each
 * [H][D] of in_dtype, rows key_stride / value_stride elements apart) into block s / B, slot s % B
 * ([Lesson06] "How paging grows").  Same dtype: bit copy.  fp8 cache: E4M3FN of float(x) /
 * scale[h], the division in binary32.  Every other byte of both pools is left unchanged. */
int orc_reshape_and_cache(void *k_pool, void *v_pool, int cache_dtype, const float *k_scale,
                          const float *v_scale, int num_blocks, int H, int D, int B,
                          const void *key, const void *value, int in_dtype, int64_t key_stride,
                          int64_t value_stride, const int64_t *slots, int T) {
  int ce = orc_elem_bytes(cache_dtype), ie = orc_elem_bytes(in_dtype);
  if (!ce || !ie || in_dtype == ORC_FP8) return -2;
  if (cache_dtype != ORC_FP8 && cache_dtype != in_dtype) return -2;
  for (int t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0 || s >= (int64_t)num_blocks * B) continue;
    int b = (int)(s / B), o = (int)(s % B);
    for (int h = 0; h < H; ++h) {
      for (int i = 0; i < D; ++i) {
        size_t src_k = (size_t)t * key_stride + (size_t)h * D + i;
        size_t src_v = (size_t)t * value_stride + (size_t)h * D + i;
        size_t dk = orc_k_index(b, h, o, i, H, D, B, cache_dtype);
        size_t dv = orc_v_index(b, h, o, i, H, D, B);
        if (cache_dtype == ORC_FP8) {
          float xk = load_elem_f32(key, in_dtype, src_k) / k_scale[h];
          float xv = load_elem_f32(value, in_dtype, src_v) / v_scale[h];
          ((uint8_t *)k_pool)[dk] = orc_e4m3_from_f32(xk);
          ((uint8_t *)v_pool)[dv] = orc_e4m3_from_f32(xv);
        } else {
          memcpy((char *)k_pool + dk * ce, (const char *)key + src_k * ie, (size_t)ce);
          memcpy((char *)v_pool + dv * ce, (const char *)value + src_v * ie, (size_t)ce);
        }
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ copy_blocks replay -------- */
/* Copy-on-write clone ([Digest] "Copy-on-write: when two requests share a prefix"): for each pair
 * {src, dst} in order and each layer, every KV head of block src is copied to block dst in both
 * pools.  block_bytes = H * B * D * element bytes (one block's span in one pool).  Pairs with an id
 * outside [0, num_blocks) are skipped. */
void orc_copy_blocks(void **k_pools, void **v_pools, int num_layers, size_t block_bytes,
                     int num_blocks, const int32_t *pairs, int num_pairs) {
  for (int k = 0; k < num_pairs; ++k) {
    int src = pairs[2 * k], dst = pairs[2 * k + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    for (int l = 0; l < num_layers; ++l) {
      memcpy((char *)k_pools[l] + (size_t)dst * block_bytes,
             (const char *)k_pools[l] + (size_t)src * block_bytes, block_bytes);
      memcpy((char *)v_pools[l] + (size_t)dst * block_bytes,
             (const char *)v_pools[l] + (size_t)src * block_bytes, block_bytes);
    }
  }
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
