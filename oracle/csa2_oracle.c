/*
 * csa2_oracle.c -- plain, slow, CPU reference of the CSA2 decode hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the HIP library; it is written from
 * the pages' description of the method:
 *   [JU] jokeuncle.pages.dev, "两张架构图里藏着 890 字节" (sections 三, 四)
 *   [WG] weigao.cc, "DeepSeek V4.1 Flash：从架构到推理成本" (sections 3.1, 3.2, 10)
 *   [SY] syt-nju.github.io, "DeepSeek-V4.1-Flash：为什么读输入只激活 8B，写输出要 16B"
 *        (CSA2 / Figure 4, Hierarchical Sparse Indexer / Figure 5, FP4 主 KV 缓存)
 *   [GP] ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析" (3.2, 3.3, 4.1, 7)
 *
 * Style: scalar loops, double-precision accumulation, qsort for orderings,
 * OpenMP only across independent entries / heads.  Float results are the
 * double result rounded once to float.
 *
 * Parity status of each function (pins live in tests/test_oracle_*.py):
 *   decode tables, quantiser, byte accounting, scoring, top-k, block pool,
 *   reindex, attention, cache write, RoPE, FP8 window record and ring: pinned (closed forms, library routines,
 *   brute force, invariants).  End-to-end values of a full decode step have
 *   no printed worked example on the pages: that composition is
 *   "parity unpinned" beyond the per-step pins.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FMT_E8M0 0
#define FMT_E4M3 1

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> value (bf16 is the upper half of an IEEE binary32). */
static double bf16_value(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* E2M1 nibble -> value.  Bit 3 is the sign, bits 2..1 the exponent (bias 1),
 * bit 0 the mantissa; exponent 0 is subnormal (0 or 0.5).  [JU 三 事实一] */
double oracle_e2m1(uint8_t nibble) {
  int sign = (nibble >> 3) & 1;
  int e = (nibble >> 1) & 3;
  int m = nibble & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * m;                     /* subnormal: m * 2^(1-1) * 0.5 */
  else
    mag = ldexp(1.0 + 0.5 * m, e - 1); /* (1 + m/2) * 2^(e-1) */
  return sign ? -mag : mag;
}

/* Scale byte -> value.  E8M0: 2^(b-127), 0xFF is NaN.  E4M3 (OCP E4M3FN):
 * sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is subnormal;
 * S.1111.111 is NaN; no infinities.  [GP 7 (E4M3 scale); SY FP4 主 KV 缓存] */
double oracle_scale_value(uint8_t b, int fmt) {
  if (fmt == FMT_E8M0) {
    if (b == 0xFF) return NAN;
    return ldexp(1.0, (int)b - 127);
  }
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 15;
  int m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* Largest finite positive scale code of a format. */
static int max_scale_code(int fmt) { return fmt == FMT_E8M0 ? 254 : 0x7E; }

/* ------------------------------------------------------------------------ */
/* Quantiser                                                                 */
/* ------------------------------------------------------------------------ */

static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* One group of n values -> n/2 code bytes + 1 scale byte.
 * The pages fix the format (E2M1 values, one scale byte per group) [JU 三;
 * GP 7] and bound the data by 6 x the largest scale; the rounding is not
 * printed, so this follows the plainest reading:
 *   scale = the smallest representable s with 6*s >= max|x| (no element clips);
 *   each |x| goes to the nearest multiple-of-s E2M1 magnitude, an exact tie
 *   going to the even code; a zero magnitude is +0.                          */
void oracle_quantize_group(const float* x, int n, int fmt, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) {
    double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  int b = 0;
  if (amax > 0.0) {
    int top = max_scale_code(fmt);
    b = top; /* saturate when no scale is large enough */
    for (int c = 0; c <= top; ++c) {
      if (6.0 * oracle_scale_value((uint8_t)c, fmt) >= amax) {
        b = c;
        break;
      }
    }
  }
  *scale = (uint8_t)b;
  double s = oracle_scale_value((uint8_t)b, fmt);
  for (int i = 0; i < n / 2; ++i) codes[i] = 0;
  for (int i = 0; i < n; ++i) {
    double a = fabs((double)x[i]);
    int code = 0;
    /* a zero magnitude is +0 whatever the scale (E4M3 code 0 is a zero scale) */
    for (int c = 1; c < 8 && a > 0.0; ++c) {
      double mid = 0.5 * (E2M1_MAG[c - 1] + E2M1_MAG[c]) * s; /* exact */
      if (a > mid || (a == mid && (c % 2) == 0)) code = c;
    }
    if (code != 0 && x[i] < 0.0f) code |= 8;
    codes[i / 2] |= (uint8_t)(code << (4 * (i % 2)));
  }
}

void oracle_quantize_rows(const float* x, int64_t rows, int dim, int group, int fmt,
                          uint8_t* codes, uint8_t* scales) {
  int ng = dim / group;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int g = 0; g < ng; ++g)
      oracle_quantize_group(x + r * dim + (int64_t)g * group, group, fmt,
                            codes + r * (dim / 2) + (int64_t)g * (group / 2),
                            scales + r * ng + g);
}

/* value of element i of an FP4 row */
static double fp4_elem(const uint8_t* codes, const uint8_t* scales, int group, int fmt, int i) {
  uint8_t byte = codes[i / 2];
  uint8_t nib = (i % 2) ? (byte >> 4) : (byte & 15);
  return oracle_e2m1(nib) * oracle_scale_value(scales[i / group], fmt);
}

void oracle_dequantize_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int dim,
                            int group, int fmt, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < dim; ++i)
      out[r * dim + i] = fp4_elem(codes + r * (dim / 2), scales + r * (dim / group), group, fmt, i);
}

/* ------------------------------------------------------------------------ */
/* Compressed RoPE                                                           */
/* ------------------------------------------------------------------------ */

/* [GP 3.2] entries are rotated with RoPE of base 160000 after RMSNorm and
 * before FP4 quantisation; [GP 7] the entry keeps 448 dims without position
 * encoding and 64 with it (128 B of bf16).  Reading: the rotated dims are the
 * last 64 (448..511), taken as 32 adjacent pairs (448+2j, 449+2j) turned by
 * the angle pos * 160000^(-2j/64).  inverse != 0 turns by -pos.            */
void oracle_rope(double* x, int64_t pos, int inverse) {
  for (int j = 0; j < 32; ++j) {
    const double ang = (double)pos * pow(160000.0, -(double)(2 * j) / 64.0) * (inverse ? -1.0 : 1.0);
    const double c = cos(ang), s = sin(ang);
    const double a = x[448 + 2 * j], b = x[449 + 2 * j];
    x[448 + 2 * j] = a * c - b * s;
    x[449 + 2 * j] = a * s + b * c;
  }
}

/* ------------------------------------------------------------------------ */
/* Cache write: gated pooling, RMSNorm, FP4, indexer-K projection            */
/* ------------------------------------------------------------------------ */

/* [JU 四 item 1] pooling weights are a per-channel softmax over the m tokens of
 * a group; ratio 1 has no gate path.  [GP 3.2 (Z)] pooled latent -> RMSNorm ->
 * FP4.  [SY CSA2; GP 3.1] the indexer K is projected from the main-KV entry.
 * y_out [T/m][512] and k_out [T/m][128] (optional) receive the fp32 values
 * that are quantised. */
void oracle_cache_write(const uint16_t* latent, const uint16_t* gate, int64_t T, int m,
                        const float* gamma, float eps, const float* w_idx, int main_fmt,
                        const int64_t* rope_pos, uint8_t* main_codes, uint8_t* main_scales,
                        uint8_t* idx_codes, uint8_t* idx_scales, float* y_out, float* k_out) {
  const int D = 512, DK = 128;
  int64_t n = T / m;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    double pooled[512];
    for (int c = 0; c < D; ++c) {
      if (m == 1) {
        pooled[c] = bf16_value(latent[j * D + c]);
        continue;
      }
      double gmax = -INFINITY;
      for (int t = 0; t < m; ++t) {
        double g = bf16_value(gate[(j * m + t) * D + c]);
        if (g > gmax) gmax = g;
      }
      double num = 0.0, den = 0.0;
      for (int t = 0; t < m; ++t) {
        double e = exp(bf16_value(gate[(j * m + t) * D + c]) - gmax);
        num += e * bf16_value(latent[(j * m + t) * D + c]);
        den += e;
      }
      pooled[c] = num / den;
    }
    double ss = 0.0;
    for (int c = 0; c < D; ++c) ss += pooled[c] * pooled[c];
    double r = 1.0 / sqrt(ss / D + (double)eps);
    float y[512];
    for (int c = 0; c < D; ++c) y[c] = (float)(pooled[c] * r * (gamma ? (double)gamma[c] : 1.0));
    /* the indexer key is projected from the entry without position encoding
     * (reading of [GP 3.2]'s "no-RoPE version"); the main entry is rotated */
    float ym[512];
    if (rope_pos) {
      double yr[512];
      for (int c = 0; c < D; ++c) yr[c] = (double)y[c];
      oracle_rope(yr, rope_pos[j], 0);
      for (int c = 0; c < D; ++c) ym[c] = (float)yr[c];
    } else {
      memcpy(ym, y, sizeof y);
    }
    float k[128];
    for (int d = 0; d < DK; ++d) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += (double)y[c] * (double)w_idx[(int64_t)c * DK + d];
      k[d] = (float)acc;
    }
    for (int g = 0; g < D / 16; ++g)
      oracle_quantize_group(ym + g * 16, 16, main_fmt, main_codes + j * 256 + g * 8,
                            main_scales + j * 32 + g);
    for (int g = 0; g < DK / 32; ++g)
      oracle_quantize_group(k + g * 32, 32, FMT_E8M0, idx_codes + j * 64 + g * 16,
                            idx_scales + j * 4 + g);
    if (y_out) memcpy(y_out + j * D, ym, sizeof ym);
    if (k_out) memcpy(k_out + j * DK, k, sizeof k);
  }
}

/* ------------------------------------------------------------------------ */
/* FP8 sliding-window record                                                  */
/* ------------------------------------------------------------------------ */

/* [GP 4.1] each layer keeps a 128-token window whose entries stay in FP8
 * (they are more sensitive to quantisation than the compressed entries);
 * [GP 7] a record is 448 B of position-free dims + 128 B of RoPE dims + 8 B
 * of scale = 584 B per token, paged with 576-B alignment; [WG 10.1] the FP8
 * window record is kept when the compressed cache is FP4; [JU 顺便算清另外三笔账]
 * the window cache has a constant 128 slots per sequence, overwritten as a
 * ring.  Readings (the byte counts are the pages'; the rest is the plainest
 * reading that fits them):
 *   - dims 0..447: OCP E4M3 codes (bias 7, largest finite 448, the value
 *     [GP 7] multiplies by 6 for its range argument), one UE8M0 scale byte per
 *     64 dims: 7 bytes, then one zero pad byte = the 8 B of scale;
 *   - dims 448..511: bf16 (64 x 2 B = the 128 B of RoPE dims);
 *   - a slot's 576 data bytes sit at a 576-B stride, its 8 scale bytes in a
 *     plane of their own;
 *   - scale = the smallest 2^(b-127) with 448*scale >= max|x| of the 64 dims
 *     (b = 0 for an all-zero group); each x/scale goes to the nearest E4M3
 *     value, an exact tie to the even code; a zero magnitude is +0;
 *   - bf16 dims are the value rounded to nearest, ties to even. */

/* nearest bf16 of a finite float, ties to the even pattern */
static uint16_t bf16_nearest(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  uint16_t lo = (uint16_t)(u >> 16); /* toward zero */
  uint16_t hi = (uint16_t)(lo + 1);  /* next magnitude up */
  double dl = fabs((double)x - bf16_value(lo)), dh = fabs(bf16_value(hi) - (double)x);
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo;
}

/* 64 values -> 64 E4M3 codes + 1 UE8M0 scale byte */
static void fp8_group(const float* x, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 64; ++i)
    if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
  int b = 0;
  if (amax > 0.0) {
    b = 254;
    for (int c = 0; c <= 254; ++c)
      if (448.0 * ldexp(1.0, c - 127) >= amax) {
        b = c;
        break;
      }
  }
  *scale = (uint8_t)b;
  const double s = ldexp(1.0, b - 127);
  for (int i = 0; i < 64; ++i) {
    const double a = fabs((double)x[i]);
    int code = 0;
    /* codes 0..126 are the finite magnitudes in increasing order */
    for (int c = 1; c <= 126 && a > 0.0; ++c) {
      const double mid = 0.5 * (oracle_scale_value((uint8_t)(c - 1), FMT_E4M3) +
                                oracle_scale_value((uint8_t)c, FMT_E4M3)) * s;
      if (a > mid || (a == mid && (c % 2) == 0)) code = c;
    }
    if (code != 0 && x[i] < 0.0f) code |= 0x80;
    codes[i] = (uint8_t)code;
  }
}

/* one 512-dim float row -> 576 data bytes + 8 scale bytes */
void oracle_fp8_record(const float* y, uint8_t* data, uint8_t* scales) {
  for (int g = 0; g < 7; ++g) fp8_group(y + 64 * g, data + 64 * g, scales + g);
  scales[7] = 0;
  for (int d = 448; d < 512; ++d) {
    const uint16_t h = bf16_nearest(y[d]);
    data[448 + 2 * (d - 448)] = (uint8_t)(h & 0xFF);
    data[449 + 2 * (d - 448)] = (uint8_t)(h >> 8);
  }
}

/* value of dim d of a record */
static double fp8_record_elem(const uint8_t* data, const uint8_t* scales, int d) {
  if (d < 448) return oracle_scale_value(data[d], FMT_E4M3) * ldexp(1.0, (int)scales[d / 64] - 127);
  const int j = 448 + 2 * (d - 448);
  return bf16_value((uint16_t)(data[j] | (data[j + 1] << 8)));
}

void oracle_fp8_record_decode(const uint8_t* data, const uint8_t* scales, int64_t rows, double* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int d = 0; d < 512; ++d) out[r * 512 + d] = fp8_record_elem(data + r * 576, scales + r * 8, d);
}

/* Window write: token i of sequence b (position pos0[b] + i) is the RMS-
 * normalised latent (the cache write's m = 1 arithmetic: no pooling), rotated
 * by the compressed RoPE at its position when rope != 0, stored as a record
 * in slot (position mod W).  Tokens are written in order, so a later token
 * overwrites an earlier one in the same slot.  swa_len[b] = min(pos0[b] + n, W):
 * the window then holds the last min(pos0[b] + n, W) tokens.
 * latent: bf16 [B][n][512]; data [B][W][576]; scales [B][W][8];
 * y_out (or NULL): float [B][n][512], the rows before FP8. */
void oracle_window_write(const uint16_t* latent, int64_t B, int n, const float* gamma, float eps,
                         int rope, const int64_t* pos0, int W, uint8_t* data, uint8_t* scales,
                         int32_t* swa_len, float* y_out) {
  const int D = 512;
  for (int64_t b = 0; b < B; ++b) {
    for (int i = 0; i < n; ++i) {
      const uint16_t* x = latent + (b * n + i) * D;
      const int64_t p = pos0[b] + i;
      double ss = 0.0;
      for (int c = 0; c < D; ++c) ss += bf16_value(x[c]) * bf16_value(x[c]);
      const double r = 1.0 / sqrt(ss / D + (double)eps);
      float y[512];
      for (int c = 0; c < D; ++c) y[c] = (float)(bf16_value(x[c]) * r * (gamma ? (double)gamma[c] : 1.0));
      if (rope) {
        double yr[512];
        for (int c = 0; c < D; ++c) yr[c] = (double)y[c];
        oracle_rope(yr, p, 0);
        for (int c = 0; c < D; ++c) y[c] = (float)yr[c];
      }
      const int64_t slot = p % W;
      oracle_fp8_record(y, data + (b * W + slot) * 576, scales + (b * W + slot) * 8);
      if (y_out) memcpy(y_out + (b * n + i) * D, y, sizeof y);
    }
    swa_len[b] = (int32_t)(pos0[b] + n < W ? pos0[b] + n : W);
  }
}

/* ------------------------------------------------------------------------ */
/* Indexer scoring                                                            */
/* ------------------------------------------------------------------------ */

/* score(p) = sum_h w_h * max(0, q_h . deq(K_p)) over H heads of 128 dims
 * (the formula stated with the tiny Full-layer workload; the pages give the
 * indexer's role but not its formula: [GP 3.3; SY Figure 5]).
 * pos: positions to score (NULL = 0..n-1); entries that are < 0 get NAN.   */
void oracle_score(const uint8_t* idx_codes, const uint8_t* idx_scales, const int32_t* pos,
                  int64_t n, const uint16_t* q, const float* w, int H, float* scores) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t p = pos ? pos[i] : i;
    if (p < 0) {
      scores[i] = NAN;
      continue;
    }
    double k[128];
    for (int d = 0; d < 128; ++d) k[d] = fp4_elem(idx_codes + p * 64, idx_scales + p * 4, 32, FMT_E8M0, d);
    double s = 0.0;
    for (int h = 0; h < H; ++h) {
      double dot = 0.0;
      for (int d = 0; d < 128; ++d) dot += bf16_value(q[h * 128 + d]) * k[d];
      s += (double)w[h] * (dot > 0.0 ? dot : 0.0);
    }
    scores[i] = (float)s;
  }
}

/* ------------------------------------------------------------------------ */
/* Selections                                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  float score;
  int64_t id;
} ranked;

/* higher score first; equal scores: lower id first */
static int rank_cmp(const void* a, const void* b) {
  const ranked* x = (const ranked*)a;
  const ranked* y = (const ranked*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int id_cmp(const void* a, const void* b) {
  int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
  return (x < y) ? -1 : (x > y);
}

/* Top-k of n (score, id) pairs by (score desc, id asc).  Writes the chosen ids
 * in ascending order into out[0..k), -1 padded; returns the number chosen.
 * Entries with NAN score are absent.  [GP 3.3: position top-512] */
int64_t oracle_topk_ids(const float* scores, const int64_t* ids, int64_t n, int64_t k,
                        int64_t* out) {
  ranked* r = (ranked*)malloc(sizeof(ranked) * (n > 0 ? n : 1));
  int64_t nv = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(scores[i])) continue;
    r[nv].score = scores[i];
    r[nv].id = ids ? ids[i] : i;
    ++nv;
  }
  qsort(r, nv, sizeof(ranked), rank_cmp);
  int64_t take = nv < k ? nv : k;
  for (int64_t i = 0; i < take; ++i) out[i] = r[i].id;
  qsort(out, take, sizeof(int64_t), id_cmp);
  for (int64_t i = take; i < k; ++i) out[i] = -1;
  free(r);
  return take;
}

/* Block maxima and candidate pool.  Block i covers [block*i, block*i+block)
 * clipped to [0, len); its score is the largest member score, an upper bound
 * of every member [GP 3.3].  The n_blocks best blocks (ties: lower block) are
 * expanded to their positions, ascending [SY Figure 5 (middle)].
 * bscore: out [ceil(len/block)] (optional).  pool: out [n_blocks*block].   */
int64_t oracle_block_pool(const float* scores, int64_t len, int block, int n_blocks,
                          float* bscore, int32_t* pool) {
  int64_t nb = (len + block - 1) / block;
  float* bs = (float*)malloc(sizeof(float) * (nb > 0 ? nb : 1));
  for (int64_t i = 0; i < nb; ++i) {
    float mx = -INFINITY;
    for (int64_t p = i * block; p < (i + 1) * block && p < len; ++p)
      if (scores[p] > mx) mx = scores[p];
    bs[i] = mx;
    if (bscore) bscore[i] = mx;
  }
  int64_t* chosen = (int64_t*)malloc(sizeof(int64_t) * (n_blocks > 0 ? n_blocks : 1));
  int64_t nch = oracle_topk_ids(bs, NULL, nb, n_blocks, chosen);
  int64_t np = 0;
  for (int64_t c = 0; c < nch; ++c)
    for (int64_t p = chosen[c] * block; p < (chosen[c] + 1) * block && p < len; ++p) pool[np++] = (int32_t)p;
  for (int64_t i = np; i < (int64_t)n_blocks * block; ++i) pool[i] = -1;
  free(chosen);
  free(bs);
  return np;
}

/* Full-mode indexer for one sequence: score every p < len once, then both the
 * position top-k and the block pool from those same scores [GP 3.3: the two
 * top-k selections share one scoring].  topk [k] int32; pool [n_blocks*block];
 * returns pool_len.  scores_out [len] optional. */
int64_t oracle_index_full(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t len,
                          const uint16_t* q, const float* w, int H, int k, int block,
                          int n_blocks, int32_t* topk, int32_t* pool, float* scores_out) {
  float* s = (float*)malloc(sizeof(float) * (len > 0 ? len : 1));
  oracle_score(idx_codes, idx_scales, NULL, len, q, w, H, s);
  int64_t* t = (int64_t*)malloc(sizeof(int64_t) * k);
  oracle_topk_ids(s, NULL, len, k, t);
  for (int i = 0; i < k; ++i) topk[i] = (int32_t)t[i];
  int64_t pl = 0;
  if (n_blocks > 0) pl = oracle_block_pool(s, len, block, n_blocks, NULL, pool);
  if (scores_out) memcpy(scores_out, s, sizeof(float) * len);
  free(t);
  free(s);
  return pl;
}

/* Reindex mode for one sequence: the layer's own (q, w) rescore only the pool
 * positions (i < pool_len; -1 or >= len masked), then top-k with ties to the
 * lower position [SY Figure 5 (right); GP 3.3].  pool_scores [pool_len] opt. */
void oracle_index_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t len,
                       const int32_t* pool, int64_t pool_len, const uint16_t* q, const float* w,
                       int H, int k, int32_t* topk, float* pool_scores) {
  int64_t n = pool_len;
  int32_t* pv = (int32_t*)malloc(sizeof(int32_t) * (n > 0 ? n : 1));
  int64_t* ids = (int64_t*)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    pv[i] = (pool[i] >= 0 && pool[i] < len) ? pool[i] : -1;
    ids[i] = pv[i];
  }
  float* s = (float*)malloc(sizeof(float) * (n > 0 ? n : 1));
  oracle_score(idx_codes, idx_scales, pv, n, q, w, H, s);
  int64_t* t = (int64_t*)malloc(sizeof(int64_t) * k);
  oracle_topk_ids(s, ids, n, k, t);
  for (int i = 0; i < k; ++i) topk[i] = (int32_t)t[i];
  if (pool_scores) memcpy(pool_scores, s, sizeof(float) * n);
  free(t);
  free(s);
  free(ids);
  free(pv);
}

/* ------------------------------------------------------------------------ */
/* Sparse attention                                                           */
/* ------------------------------------------------------------------------ */

/* Core attention of one query of H heads x 512 dims [SY CSA2 Figure 4]: the
 * selected main-KV entries (topk j with 0 <= topk[j] < len) concatenated with
 * swa_len window entries; rows are dequantised first [SY FP4 主 KV 缓存] and act
 * as both key and value.  out [H][512] fp32; lse [H] (optional).             */
void oracle_attention(const uint16_t* q, int H, const uint8_t* main_codes,
                      const uint8_t* main_scales, int64_t len, int main_fmt,
                      const int32_t* topk, int k, const uint8_t* swa_codes,
                      const uint8_t* swa_scales, int swa_len, int swa_fmt, float sm_scale,
                      const int64_t* q_pos, float* out, float* lse) {
  const int D = 512;
  int nrow = 0;
  for (int j = 0; j < k; ++j)
    if (topk[j] >= 0 && topk[j] < len) ++nrow;
  nrow += swa_len;
  double* rows = (double*)malloc(sizeof(double) * D * (nrow > 0 ? nrow : 1));
  int r = 0;
  for (int j = 0; j < k; ++j) {
    if (!(topk[j] >= 0 && topk[j] < len)) continue;
    int64_t p = topk[j];
    for (int d = 0; d < D; ++d)
      rows[(int64_t)r * D + d] = fp4_elem(main_codes + p * 256, main_scales + p * 32, 16, main_fmt, d);
    ++r;
  }
  /* window rows: the main format (swa_fmt 0) or FP8 records (swa_fmt 1) */
  for (int j = 0; j < swa_len; ++j, ++r)
    for (int d = 0; d < D; ++d)
      rows[(int64_t)r * D + d] =
          swa_fmt ? fp8_record_elem(swa_codes + (int64_t)j * 576, swa_scales + (int64_t)j * 8, d)
                  : fp4_elem(swa_codes + (int64_t)j * 256, swa_scales + (int64_t)j * 32, 16, main_fmt, d);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h) {
    double* logit = (double*)malloc(sizeof(double) * (nrow > 0 ? nrow : 1));
    /* [WG 10] vLLM's fused decode path rotates the query (Q RoPE) and
     * turns the output back (inverse RoPE); reading: both at the query's
     * position, on the same 64 dims as the entries */
    double qh[512];
    for (int d = 0; d < D; ++d) qh[d] = bf16_value(q[(int64_t)h * D + d]);
    if (q_pos) oracle_rope(qh, *q_pos, 0);
    double mx = -INFINITY;
    for (int j = 0; j < nrow; ++j) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += qh[d] * rows[(int64_t)j * D + d];
      logit[j] = (double)sm_scale * dot;
      if (logit[j] > mx) mx = logit[j];
    }
    double den = 0.0;
    for (int j = 0; j < nrow; ++j) den += exp(logit[j] - mx);
    double o[512];
    for (int d = 0; d < D; ++d) {
      double acc = 0.0;
      for (int j = 0; j < nrow; ++j) acc += exp(logit[j] - mx) * rows[(int64_t)j * D + d];
      o[d] = nrow > 0 ? acc / den : 0.0;
    }
    if (q_pos) oracle_rope(o, *q_pos, 1);
    for (int d = 0; d < D; ++d) out[(int64_t)h * D + d] = (float)o[d];
    if (lse) lse[h] = nrow > 0 ? (float)(mx + log(den)) : -INFINITY;
    free(logit);
  }
  free(rows);
}

/* Threads OpenMP would use (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Set the number of OpenMP threads of later calls (timing of the oracle on
 * one core beside all cores; no effect on any result). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
