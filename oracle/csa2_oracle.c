/*
 * CSA2 decode-path ORACLE -- test infrastructure only.
 *
 * A plain, slow CPU statement of what the CSA2 decode hot path computes.
 * Only tests/, the smoke check and the benchmark's cpu_baseline leg load it;
 * the product library never links or calls it, and it shares no code,
 * header, table or helper with the HIP path.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math), so
 * every float expression below is evaluated exactly as written, in IEEE
 * binary32/binary64 with round-to-nearest-even.
 *
 * Sources (pages under /root/reference, cited by page title and section):
 *  [P1] "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression"
 *       (knowledge note): "CSA2: share cache, refresh selection only when
 *       needed" (mode table), "Hierarchical Sparse Indexer" (Figure 5),
 *       "FP4 main KV: trade precision for bytes".
 *  [P2] "Inside DeepSeek V4.1 Flash: CED, CSA2 and the 890-Byte KV Cache":
 *       "CSA2: reuse memory and reuse selection independently",
 *       "Hierarchical indexing bounds later searches, not every search",
 *       "Reconstructing the 890-byte cache budget".
 * Where the pages leave a step open, the reading taken is named inline
 * ("reading:") and listed in the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define D_MAIN 512          /* main-KV channels [P2 890-byte budget] */
#define D_IDX 128           /* indexer-key channels [P2 890-byte budget] */
#define GROUP 16            /* channels per E4M3 scale [P1 FP4 main KV] */
#define NGROUPS (D_MAIN / GROUP)
#define PAGE 64             /* entries per cache page (paged-cache reading) */
#define ENTRY_CODES (D_MAIN / 2)               /* 256 B of E2M1 nibbles */
#define ENTRY_BYTES (ENTRY_CODES + NGROUPS)    /* 288 B [P2 budget] */
#define PAGE_BYTES (PAGE * ENTRY_BYTES)
#define BLOCK 8             /* positions per pool block [P1 Fig. 5] */

/* ---------------- O1: number formats ---------------- */

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinity.
 * Largest finite value 448. */
double csa2o_e4m3_decode(uint32_t code) {
  code &= 0xFF;
  uint32_t s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, (int)e - 10);
  return s ? -v : v;
}

/* OCP FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.
 * Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double csa2o_e2m1_decode(uint32_t code) {
  code &= 0xF;
  uint32_t s = code >> 3, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return s ? -v : v;
}

/* bf16 -> binary64, exact (bf16 is the top half of a binary32). */
double csa2o_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Nearest positive finite E4M3 code to t = num/6, ties to the even code,
 * saturating at 448 (code 0x7E).  Written as a plain search over all 127
 * non-negative finite codes.  Distances |num - 6 v| are exact in binary64
 * (num is a bf16 value, 6 v has at most 6 significant bits), so comparing
 * them is comparing |t - v| exactly without ever forming t. */
uint32_t csa2o_e4m3_nearest_sixth(double num) {
  uint32_t best = 0;
  double bestd = INFINITY;
  for (uint32_t c = 0; c <= 0x7E; ++c) {
    double d = fabs(num - 6.0 * csa2o_e4m3_decode(c));
    if (d < bestd || (d == bestd && (c & 1) == 0)) {
      bestd = d;
      best = c;
    }
  }
  return best;
}

/* Nearest E4M3 code to x (any sign), ties to even, saturating to +-448.
 * Used by tests to pin the search against the format definition. */
uint32_t csa2o_e4m3_nearest(double x) {
  uint32_t mag = csa2o_e4m3_nearest_sixth(6.0 * fabs(x));
  return (signbit(x) ? 0x80u : 0u) | mag;
}

/* Nearest E2M1 magnitude code to a / s (a >= 0, s > 0), ties to the even
 * code, saturating at 6 (code 7).  Distances |a - s g| are exact in binary64
 * (a is bf16, s g has at most 6 significant bits). */
uint32_t csa2o_e2m1_nearest(double a, double s) {
  uint32_t best = 0;
  double bestd = INFINITY;
  for (uint32_t m = 0; m < 8; ++m) {
    double d = fabs(a - s * csa2o_e2m1_decode(m));
    if (d < bestd || (d == bestd && (m & 1) == 0)) {
      bestd = d;
      best = m;
    }
  }
  return best;
}

/* ---------------- O2: FP4 main-KV cache write ----------------
 * [P1 FP4 main KV] and [P2 890-byte budget]: E2M1 elements with one E4M3
 * scale per 16 channels, no second-level global scale; 512 channels give
 * 256 B of codes + 32 B of scales = 288 B per entry.
 * Readings: the scale is the E4M3 value nearest to amax/6 (6 = largest E2M1
 * magnitude), ties to even, saturating; each element is the E2M1 value
 * nearest to |x|/scale with the sign of x copied (also for -0 and for values
 * that round to zero); a zero scale gives zero magnitudes; channel 2i sits
 * in the low nibble of byte i. */
void csa2o_quantize_row(const uint16_t *x, uint8_t *codes, uint8_t *scales) {
  memset(codes, 0, ENTRY_CODES);
  for (int g = 0; g < NGROUPS; ++g) {
    double amax = 0.0;
    for (int c = 0; c < GROUP; ++c) {
      double v = fabs(csa2o_bf16_to_double(x[g * GROUP + c]));
      if (v > amax) amax = v;
    }
    uint32_t sc = csa2o_e4m3_nearest_sixth(amax);
    double s = csa2o_e4m3_decode(sc);
    scales[g] = (uint8_t)sc;
    for (int c = 0; c < GROUP; ++c) {
      int ch = g * GROUP + c;
      uint16_t h = x[ch];
      double a = fabs(csa2o_bf16_to_double(h));
      uint32_t m = (s > 0.0) ? csa2o_e2m1_nearest(a, s) : 0u;
      uint32_t code = ((uint32_t)(h >> 15) << 3) | m;
      codes[ch / 2] |= (uint8_t)((ch & 1) ? (code << 4) : code);
    }
  }
}

/* Many rows at once: the same per-row statement, rows in parallel. */
void csa2o_quantize_rows(const uint16_t *x, int64_t rows, uint8_t *codes, uint8_t *scales) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    csa2o_quantize_row(x + r * D_MAIN, codes + r * ENTRY_CODES, scales + r * NGROUPS);
}

/* Paged cache write.  Reading of the page layout: a page holds 64 entries,
 * first their 64 x 256 B of codes, then their 64 x 32 B of scales; row r is
 * written to slot dst_slot[r] = page * 64 + offset.  Rows whose slot falls
 * outside the pool are not written. */
void csa2o_quantize_kv(const uint16_t *x, int64_t rows, const int64_t *dst_slot,
                       uint8_t *pool, int64_t n_pages) {
  for (int64_t r = 0; r < rows; ++r) {
    int64_t slot = dst_slot[r];
    if (slot < 0 || slot >= n_pages * PAGE) continue;
    int64_t page = slot / PAGE, off = slot % PAGE;
    uint8_t *base = pool + page * PAGE_BYTES;
    csa2o_quantize_row(x + r * D_MAIN, base + off * ENTRY_CODES,
                       base + PAGE * ENTRY_CODES + off * NGROUPS);
  }
}

/* ---------------- O3: dequantize-at-use ----------------
 * [P1 FP4 main KV]: the cache is widened before attention.  x = E2M1 * s,
 * exact in binary64. */
void csa2o_dequant_entry(const uint8_t *codes, const uint8_t *scales, double *out) {
  for (int ch = 0; ch < D_MAIN; ++ch) {
    uint32_t nib = (ch & 1) ? (codes[ch / 2] >> 4) : (codes[ch / 2] & 0xF);
    out[ch] = csa2o_e2m1_decode(nib) * csa2o_e4m3_decode(scales[ch / GROUP]);
  }
}

void csa2o_dequant_rows(const uint8_t *codes, const uint8_t *scales, int64_t rows, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    csa2o_dequant_entry(codes + r * ENTRY_CODES, scales + r * NGROUPS, out + r * D_MAIN);
}

/* ---------------- O4: indexer score ----------------
 * [P1 Hierarchical Sparse Indexer], [P2 CSA2 modes]: a lightweight indexer
 * scores each compressed position with the layer's indexer query against the
 * shared indexer key.  The pages print no formula.  Reading (lightning-
 * indexer lineage named on [P1]): per indexer head h,
 *   d_h = sum_c q[h][c] * k[c]            (exact, then rounded once to fp32)
 *   r_h = d_h > 0 ? d_h : +0
 *   t_h = fl(w_h r_h) for h < H, t_h = +0 for H <= h < 64 (H <= 64)
 *   s   = pairwise(t_0 .. t_63) + 0
 * where pairwise() is the balanced binary tree over the 64 slots in
 * ascending order: ((t_0 + t_1) + (t_2 + t_3)) + ..., every multiply and
 * add a separate binary32 operation; the final + 0 turns -0 into +0.  The
 * pages leave the order of the head sum open; a pairwise tree is the order
 * a parallel reduction takes.  Each product of two E4M3 values is a multiple of 2^-18
 * below 2^18, so any sum of 128 of them fits in 43 bits and the binary64
 * accumulation below is exact; the cast to float is the single rounding.
 * q: [H][128] E4M3 codes; keys: [n][128] E4M3 codes; s: [n]. */
void csa2o_index_scores(const uint8_t *q, const float *w, int H,
                        const uint8_t *keys, int64_t n, float *s) {
  double qv[64 * D_IDX];
  double (*qd)[D_IDX] = (double (*)[D_IDX])qv;
  if (H < 0 || H > 64) { /* the sum has 64 slots: more heads are not defined */
    for (int64_t j = 0; j < n; ++j) s[j] = NAN;
    return;
  }
  for (int h = 0; h < H; ++h)
    for (int c = 0; c < D_IDX; ++c) qd[h][c] = csa2o_e4m3_decode(q[h * D_IDX + c]);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    double kd[D_IDX];
    for (int c = 0; c < D_IDX; ++c) kd[c] = csa2o_e4m3_decode(keys[j * D_IDX + c]);
    float t[64];
    for (int h = 0; h < 64; ++h) {
      t[h] = 0.0f;
      if (h >= H) continue;
      double dot = 0.0;
      for (int c = 0; c < D_IDX; ++c) dot += qd[h][c] * kd[c];
      float d = (float)dot;
      float r = d > 0.0f ? d : 0.0f;
      t[h] = w[h] * r;
    }
    for (int width = 32; width >= 1; width /= 2)
      for (int i = 0; i < width; ++i) t[i] = t[2 * i] + t[2 * i + 1];
    s[j] = t[0] + 0.0f;
  }
}

/* ---------------- O5: top-k ----------------
 * Keep the k best positions.  Reading (ties broken toward the lower index):
 * rank by (score descending, index ascending), keep min(k, n), write the
 * kept indices in ascending order and pad with -1.  idx[i] is the global
 * index of candidate i (ties use it). */
typedef struct {
  float s;
  int32_t j;
} scored_t;

static int cmp_rank(const void *a, const void *b) {
  const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

void csa2o_topk(const float *s, const int32_t *idx, int64_t n, int32_t k, int32_t *out) {
  scored_t *v = (scored_t *)malloc(sizeof(scored_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    v[i].s = s[i];
    v[i].j = idx ? idx[i] : (int32_t)i;
  }
  qsort(v, (size_t)n, sizeof(scored_t), cmp_rank);
  int64_t keep = n < k ? n : k;
  for (int64_t i = 0; i < keep; ++i) out[i] = v[i].j;
  qsort(out, (size_t)keep, sizeof(int32_t), cmp_i32);
  for (int64_t i = keep; i < k; ++i) out[i] = -1;
  free(v);
}

/* ---------------- O6: block-max candidate pool ----------------
 * [P1 Hierarchical Sparse Indexer, Fig. 5], [P2 hierarchical indexing]: the
 * Full layer scores blocks of 8 positions by their maximum position score
 * and keeps up to 2,048 blocks (<= 16,384 positions).  Reading: block b is
 * positions [8b, 8b+8) clipped to n; rank blocks by (block score desc,
 * block id asc); keep min(pool_blocks, n_blocks); write ascending, pad -1. */
void csa2o_pool(const float *s, int64_t n, int32_t pool_blocks, int32_t *out_blocks,
                int32_t *out_n) {
  int64_t nb = (n + BLOCK - 1) / BLOCK;
  float *bs = (float *)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1));
  for (int64_t b = 0; b < nb; ++b) {
    float m = s[b * BLOCK];
    for (int64_t j = b * BLOCK + 1; j < n && j < (b + 1) * BLOCK; ++j)
      if (s[j] > m) m = s[j];
    bs[b] = m;
  }
  csa2o_topk(bs, NULL, nb, pool_blocks, out_blocks);
  *out_n = (int32_t)(nb < pool_blocks ? nb : pool_blocks);
  free(bs);
}

/* ---------------- O9: attention over selected entries + local window ----
 * [P2 CSA2]: the main query attends to the selected global entries together
 * with the local sliding window; [P1 FP4 main KV] the global entries are
 * dequantized first; the window is FP8.  Readings: one softmax over the
 * union of rows, the 512-channel entry serves as both key and value,
 * logits are sm_scale * q . row.  Evaluated in binary64.
 * q: [H][512]; rows: [nr][512]; out: [H][512]; lse: [H] (natural log). */
void csa2o_attention(const double *q, int H, double sm_scale, const double *rows,
                     int64_t nr, double *out, double *lse) {
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    double *l = (double *)malloc(sizeof(double) * (size_t)(nr > 0 ? nr : 1));
    double mx = -INFINITY;
    for (int64_t r = 0; r < nr; ++r) {
      double dot = 0.0;
      for (int c = 0; c < D_MAIN; ++c) dot += q[h * D_MAIN + c] * rows[r * D_MAIN + c];
      l[r] = sm_scale * dot;
      if (l[r] > mx) mx = l[r];
    }
    double z = 0.0;
    for (int64_t r = 0; r < nr; ++r) {
      l[r] = exp(l[r] - mx);
      z += l[r];
    }
    for (int c = 0; c < D_MAIN; ++c) {
      double acc = 0.0;
      for (int64_t r = 0; r < nr; ++r) acc += l[r] * rows[r * D_MAIN + c];
      out[h * D_MAIN + c] = acc / z;
    }
    if (lse) lse[h] = mx + log(z);
    free(l);
  }
}

int csa2o_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
