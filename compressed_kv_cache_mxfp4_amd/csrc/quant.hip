// quant.hip -- FP4 quantiser and the KV-source cache write (gfx950).
//
// Format [jokeuncle.pages.dev, "两张架构图里藏着 890 字节", section 三 (事实一, 事实二);
// ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析", section 7]:
// E2M1 values, one scale byte per group (16 for the main KV with an E4M3 or
// E8M0 scale, 32 for the indexer K with E8M0).  Rounding (a reading; the
// pages do not print it): the smallest scale s with 6*s >= group max, then
// round-to-nearest E2M1, ties to the even code, zero magnitude -> +0.
//
// The cache write follows [jokeuncle.pages.dev, section 四 item 1] (per-channel
// softmax pooling over the m tokens of a group, fp32 when m > 1),
// [ggaaooppeenngg.github.io, section 3.2 "Z"] (pooled -> RMSNorm -> FP4) and
// [syt-nju.github.io, "为什么读输入只激活 8B", section CSA2] (indexer K projected
// from the main-KV entry).  With entry positions given, the main entry's
// dims 448..511 are rotated by the compressed RoPE before FP4 [same
// ggaaooppeenngg.github.io page, 3.2]; the indexer key is projected from the
// entry before rotation.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

// ---------------------------------------------------------------- scale rule
__device__ __forceinline__ uint32_t scale_code_e8m0(float amax) {
  if (!(amax > 0.0f)) return 0u;
  uint32_t u = __float_as_uint(amax);
  int eb = (int)(u >> 23);
  if (eb == 0) return 0u;      // subnormal max: 6 * 2^-127 already covers it
  if (eb >= 255) return 254u;  // inf: saturate
  // amax = f * 2^(eb-127), f in [1,2): need 2^(b-127) >= f/6 * 2^(eb-127)
  int b = eb - 2 + ((u & 0x7FFFFFu) > 0x400000u ? 1 : 0);
  b = b < 0 ? 0 : (b > 254 ? 254 : b);
  return (uint32_t)b;
}

// Smallest E4M3 code b (0x7E at most) with 6 * value(b) >= amax, in closed
// form: t = amax * RN(1/6) taken up to the E4M3 grid -- m * 2^-9 below 2^-6,
// else the exponent and three fraction bits rounded up -- then one code up if
// 6 * value(b) < amax (an exact test: 6 * value(b) has at most five
// significant bits).  t never rounds past a grid value v with 6 v >= amax:
// 6 RN(1/6) - 1 < 2^-25, so amax RN(1/6) <= v (1 + 2^-25) stays within half
// an ulp of v (v's significand is at most 1.875).  It can fall below amax / 6
// by half an ulp, hence the one step up.  Equal to a search over the codes
// for every non-NaN fp32 amax (checked exhaustively on the host).
__device__ __forceinline__ uint32_t scale_code_e4m3(float amax) {
  if (!(amax > 0.0f)) return 0u;
  const float t = amax * (1.0f / 6.0f);
  int b = t < 0x1p-6f ? (int)ceilf(t * 512.0f) : (int)((__float_as_uint(t) - (120u << 23) + 0xFFFFFu) >> 20);
  b = min(b, 0x7E);
  if (6.0f * e4m3_value((uint32_t)b) < amax) b = min(b + 1, 0x7E);
  return (uint32_t)b;
}

template <int FMT>
__device__ __forceinline__ uint32_t scale_code(float amax) {
  return FMT == 0 ? scale_code_e8m0(amax) : scale_code_e4m3(amax);
}

template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t b) {
  return FMT == 0 ? e8m0_value(b) : e4m3_value(b);
}

// The encoding rule: the nearest E2M1 code of x / s, ties to the even code,
// saturating at 6, a zero magnitude as +0 and NaN as 0.  gfx950's
// v_cvt_scalef32_pk_fp4_f32 applies it for power-of-two scales, two values
// per instruction; other scales are divided out first (E4M3 below).

// E2M1 codes of values over a power-of-two scale s (an E8M0 value), two per
// v_cvt_scalef32_pk_fp4_f32: x / s rounded to nearest, ties to even,
// saturating at 6 -- measured on gfx950 to agree with the rule for every
// midpoint and its neighbours, every grid point, saturation, subnormal values
// and subnormal scales (2^-127 .. 2^30), except that it gives a zero
// magnitude the sign of x and saturates NaN.  So NaN is taken as 0 first and
// the sign of zero magnitudes is cleared after.
__device__ __forceinline__ float nan_to_zero(float x) { return x == x ? x : 0.0f; }

__device__ __forceinline__ uint32_t clear_negative_zeros(uint32_t w) {
  const uint32_t mag = w & 0x77777777u;
  return mag | (w & ((mag + 0x77777777u) & 0x88888888u));  // sign kept where the magnitude is not 0
}

// one value -> its code (low nibble)
__device__ __forceinline__ uint32_t e2m1_pow2(float x, float s) {
  return clear_negative_zeros(__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, nan_to_zero(x), 0.0f, s, 0)) & 15u;
}

// 8 values -> one code dword (value j in nibble j)
__device__ __forceinline__ uint32_t e2m1x8_pow2(const float (&v)[8], float s) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, nan_to_zero(v[0]), nan_to_zero(v[1]), s, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, nan_to_zero(v[2]), nan_to_zero(v[3]), s, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, nan_to_zero(v[4]), nan_to_zero(v[5]), s, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, nan_to_zero(v[6]), nan_to_zero(v[7]), s, 3);
  return clear_negative_zeros(w);
}

// E2M1 codes over an E4M3 scale s = 2^E * sig (sig = 1 + j/8; the subnormal
// codes' m * 2^-9 normalise the same way): the convert takes 2^E, and each
// value is first divided by sig, correctly rounded -- the product with
// r = RN(1/sig) and one residual step, q = q0 + (x - q0 sig) r, which gives
// RN(x / sig) when q0 is within an ulp and r within half an ulp (Markstein's
// theorem).  The codes follow the rule for x / s: a midpoint M of the grid (at
// most 3 significant bits) times sig has at most 7, so an fp32 x other than
// M sig 2^E has x / sig more than half an ulp of M 2^E away from it, and the
// rounded quotient stays on the same side of every midpoint; x = M sig 2^E
// gives the midpoint itself, which the convert rounds to the even code.
// Checked on the host for every fp32 x in [s 2^-7, s 2^5) and every scale
// code.  NaN is taken as 0 and infinities are clamped to +-2^100 (still
// saturating) so that the residual stays finite.  Scale code 0 (a group of
// zeros) converts at 2^0.
struct E4m3Div {
  float sig, r, pow2;
};

__device__ __forceinline__ E4m3Div e4m3_div(float s) {
  const uint32_t su = __float_as_uint(s);
  const float sig = __uint_as_float((su & 0x007FFFFFu) | 0x3F800000u);
  return E4m3Div{sig, 1.0f / sig, s == 0.0f ? 1.0f : __uint_as_float(su & 0x7F800000u)};
}

__device__ __forceinline__ float e4m3_quot(float x, const E4m3Div& d) {
  const float xc = fminf(fmaxf(nan_to_zero(x), -0x1p100f), 0x1p100f);
  const float q0 = xc * d.r;
  return fmaf(fmaf(-q0, d.sig, xc), d.r, q0);
}

__device__ __forceinline__ uint32_t e2m1x8_e4m3(const float (&v)[8], float s) {
  const E4m3Div d = e4m3_div(s);
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, e4m3_quot(v[0], d), e4m3_quot(v[1], d), d.pow2, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e4m3_quot(v[2], d), e4m3_quot(v[3], d), d.pow2, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e4m3_quot(v[4], d), e4m3_quot(v[5], d), d.pow2, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e4m3_quot(v[6], d), e4m3_quot(v[7], d), d.pow2, 3);
  return clear_negative_zeros(w);
}

// 8 values -> one code dword with the group's scale s of format FMT
template <int FMT>
__device__ __forceinline__ uint32_t e2m1x8(const float (&v)[8], float s) {
  if constexpr (FMT == 0)
    return e2m1x8_pow2(v, s);
  else
    return e2m1x8_e4m3(v, s);
}

// Softmax pooling of a channel over two tokens (m = 2): the token with the
// larger gate weighs 1 / (1 + e) and the other e / (1 + e), e = exp(-|g0 -
// g1|) -- the rule's weights exp(g_t - max) / sum, whose larger term is
// exp(0) = 1, so one exponential per channel.  e is exp2 of -|g0 - g1| log2 e
// (v_exp_f32, 1 ulp; the product's rounding moves e by about |g0 - g1|
// 2^-24 relative) and the quotient a hardware reciprocal: a few ulps of fp32
// in all.  A gate of +inf gives NaN (exp(inf - inf)), as do NaN gates and
// two -inf gates.
__device__ __forceinline__ float pool2(float g0, float g1, float x0, float x1) {
  const float gm = fmaxf(g0, g1);
  const float e = __builtin_amdgcn_exp2f(-fabsf(g0 - g1) * 1.4426950408889634f) + (gm - gm);
  const bool first = g0 >= g1;
  const float xa = first ? x0 : x1, xb = first ? x1 : x0;
  return fmaf(e, xb, xa) * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------- generic quantiser
// One lane per 4 consecutive values; GROUP/4 lanes share a scale.
template <int GROUP, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ x, int64_t n4,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  constexpr int LPG = GROUP / 4;
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = i4 < n4;
  float4 v = active ? reinterpret_cast<const float4*>(x)[i4] : make_float4(0.f, 0.f, 0.f, 0.f);
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  amax = group_reduce<LPG, true>(amax);
  const uint32_t b = scale_code<FMT>(amax);
  const float s = scale_value<FMT>(b);
  if (!active) return;
  uint32_t c;
  if constexpr (FMT == 0) {
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, nan_to_zero(v.x), nan_to_zero(v.y), s, 0);
    c = clear_negative_zeros(__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, nan_to_zero(v.z), nan_to_zero(v.w), s, 1));
  } else {
    const E4m3Div d = e4m3_div(s);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, e4m3_quot(v.x, d), e4m3_quot(v.y, d), d.pow2, 0);
    c = clear_negative_zeros(__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, e4m3_quot(v.z, d), e4m3_quot(v.w, d), d.pow2, 1));
  }
  reinterpret_cast<uint16_t*>(codes)[i4] = (uint16_t)c;
  if ((i4 % LPG) == 0) scales[i4 / LPG] = (uint8_t)b;
}

int launch_quantize(const float* x, int64_t rows, int dim, int group, int fmt, uint8_t* codes,
                    uint8_t* scales, hipStream_t st) {
  const int64_t n4 = rows * (int64_t)dim / 4;
  if (n4 == 0) return 0;
  const int threads = 256;
  const int64_t blocks = (n4 + threads - 1) / threads;
  if (group == 16 && fmt == 0)
    quantize_kernel<16, 0><<<dim3((unsigned)blocks), threads, 0, st>>>(x, n4, codes, scales);
  else if (group == 16 && fmt == 1)
    quantize_kernel<16, 1><<<dim3((unsigned)blocks), threads, 0, st>>>(x, n4, codes, scales);
  else if (group == 32 && fmt == 0)
    quantize_kernel<32, 0><<<dim3((unsigned)blocks), threads, 0, st>>>(x, n4, codes, scales);
  else
    quantize_kernel<32, 1><<<dim3((unsigned)blocks), threads, 0, st>>>(x, n4, codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------- cache write
// A workgroup of 8 waves takes 16 entries.  Phase 1: each wave pools and
// normalises 2 entries (lane: 8 channels) into LDS and, in the workgroup of
// column split 0, quantises the main entries.  Phase 2: the indexer-K
// projection K[16 x 128] = Y[16 x 512] . W[512 x 128] on fp32 MFMA
// (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation), with W read
// once per workgroup straight into the B operands.  K step ks of lane group
// g is channel 128g + ks, so one 16-byte LDS read gives a lane its A operand
// (Y) of four consecutive steps.  The workgroup's columns form groups of
// CW = 64 (or 32): lane n of a group loads the CW/16 adjacent columns
// CW/16*n .. +CW/16-1 of one W row in one load, and MFMA j takes column
// CW/16*n + j of each lane -- a permuted 16-column tile -- so one load feeds
// CW/16 products.  The waves of a column group split its K steps, and their
// partial products are summed through LDS.  Phase 3: E8M0 FP4 of the keys.
// A workgroup covers all 128 columns when there are enough entries to fill
// the chip (T = 8 column tiles of 16); for smaller writes the columns are
// split over 8/T workgroups per entry tile (T >= 2: a workgroup holds whole
// 32-column scale groups).
constexpr int kWriteEntries = 16;  // entries per workgroup
constexpr int kWriteWaves = 8;
constexpr int kYLd = 516;          // LDS row stride of Y (fp32): conflict-free 16-byte reads
constexpr int kKLd = 132;          // LDS row stride of the projected keys

template <int FMT, int T>
__global__ __launch_bounds__(64 * kWriteWaves, 2) void cache_write_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ gate, int64_t n_entries,
    int m, const float* __restrict__ gamma, float eps, const float* __restrict__ w_idx,
    const int64_t* __restrict__ rope_pos, uint8_t* __restrict__ main_codes,
    uint8_t* __restrict__ main_scales, uint8_t* __restrict__ idx_codes,
    uint8_t* __restrict__ idx_scales) {
  // at least one whole E8M0 group (32 columns) of the indexer key per workgroup
  static_assert(T == 2 || T == 4 || T == 8, "column tiles per workgroup");
  constexpr int kCW = T == 2 ? 32 : 64;          // columns of a column group
  constexpr int kJ = kCW / 16;                   // adjacent columns per lane (and MFMAs per K step)
  constexpr int kGroups = 16 * T / kCW;          // column groups of the workgroup
  constexpr int kWpg = kWriteWaves / kGroups;    // waves per column group
  constexpr int kSteps = 128 / kWpg;             // K steps per wave
  // normalised entries (phases 1-2), then the waves' partial products (the
  // same LDS, after a barrier)
  __shared__ __align__(16) float ybuf[kWriteEntries * kYLd];
  static_assert(kWriteWaves * kJ * 256 <= kWriteEntries * kYLd, "partials fit in the entry buffer");
  float (*yS)[kYLd] = reinterpret_cast<float (*)[kYLd]>(ybuf);
  float (*part)[kJ * 256] = reinterpret_cast<float (*)[kJ * 256]>(ybuf);
  __shared__ __align__(16) float kS[kWriteEntries][kKLd];          // projected keys (16 T columns)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int cs = blockIdx.y;                 // column split: columns 16T*cs .. 16T*cs + 16T - 1
  const int64_t e0 = (int64_t)blockIdx.x * kWriteEntries;
  constexpr int kEpw = kWriteEntries / kWriteWaves;  // entries per wave

  // ---- phase 1.  Ratio 1 and 2: every latent (and gate) load of the wave
  // is issued before any arithmetic, so its entries cost one memory round trip.
  uint4 xpre[kEpw][2], gpre[kEpw][2];
  if (m <= 2) {
#pragma unroll
    for (int j = 0; j < kEpw; ++j) {
      const int64_t e = e0 + wave + kWriteWaves * j;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bool ok = e < n_entries && t < m;
        xpre[j][t] = ok ? *reinterpret_cast<const uint4*>(latent + (e * m + t) * 512 + 8 * lane)
                        : make_uint4(0u, 0u, 0u, 0u);
        gpre[j][t] = ok && m > 1 ? *reinterpret_cast<const uint4*>(gate + (e * m + t) * 512 + 8 * lane)
                                 : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  // W of this wave's first K steps in flight during the pooling
  typedef float wvec __attribute__((ext_vector_type(kJ)));
  const int grp = wave / kWpg, kr = wave % kWpg;        // column group, K range
  const int g = lane >> 4, n = lane & 15;
  const int cbase = 16 * T * cs + kCW * grp;            // first column of the group
  const int d = cbase + kJ * n;                         // this lane's first column
  const int ks0 = kr * kSteps;                          // first K step of this wave
  constexpr int kPre = kSteps < 8 ? kSteps : 8;         // W loads in flight
  wvec wpre[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) wpre[i] = *reinterpret_cast<const wvec*>(w_idx + (128 * g + ks0 + i) * 128 + d);

#pragma unroll
  for (int j = 0; j < kEpw; ++j) {
    const int ei = wave + kWriteWaves * j;
    const int64_t e = e0 + ei;
    if (e >= n_entries) {
#pragma unroll
      for (int c = 0; c < 8; ++c) yS[ei][8 * lane + c] = 0.0f;
      continue;
    }
    float pooled[8];
    if (m == 1) {
      const uint32_t xw[4] = {xpre[j][0].x, xpre[j][0].y, xpre[j][0].z, xpre[j][0].w};
#pragma unroll
      for (int c = 0; c < 8; ++c) pooled[c] = bf16_bits_to_f32((xw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
    } else if (m == 2) {
      const uint32_t g0w[4] = {gpre[j][0].x, gpre[j][0].y, gpre[j][0].z, gpre[j][0].w};
      const uint32_t g1w[4] = {gpre[j][1].x, gpre[j][1].y, gpre[j][1].z, gpre[j][1].w};
      const uint32_t x0w[4] = {xpre[j][0].x, xpre[j][0].y, xpre[j][0].z, xpre[j][0].w};
      const uint32_t x1w[4] = {xpre[j][1].x, xpre[j][1].y, xpre[j][1].z, xpre[j][1].w};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int sh = 16 * (c % 2);
        pooled[c] = pool2(bf16_bits_to_f32((g0w[c / 2] >> sh) & 0xFFFFu), bf16_bits_to_f32((g1w[c / 2] >> sh) & 0xFFFFu),
                          bf16_bits_to_f32((x0w[c / 2] >> sh) & 0xFFFFu), bf16_bits_to_f32((x1w[c / 2] >> sh) & 0xFFFFu));
      }
    } else {
      float gmax[8], num[8], den[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) { gmax[c] = -INFINITY; num[c] = 0.f; den[c] = 0.f; }
      for (int t = 0; t < m; ++t) {
        uint4 gv = *reinterpret_cast<const uint4*>(gate + (e * m + t) * 512 + 8 * lane);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) gmax[c] = fmaxf(gmax[c], bf16_bits_to_f32((gw[c / 2] >> (16 * (c % 2))) & 0xFFFFu));
      }
      for (int t = 0; t < m; ++t) {
        uint4 gv = *reinterpret_cast<const uint4*>(gate + (e * m + t) * 512 + 8 * lane);
        uint4 xv = *reinterpret_cast<const uint4*>(latent + (e * m + t) * 512 + 8 * lane);
        const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float ex = expf(bf16_bits_to_f32((gw[c / 2] >> (16 * (c % 2))) & 0xFFFFu) - gmax[c]);
          num[c] += ex * bf16_bits_to_f32((xw[c / 2] >> (16 * (c % 2))) & 0xFFFFu);
          den[c] += ex;
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) pooled[c] = num[c] / den[c];
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss += pooled[c] * pooled[c];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / 512.0f + eps);
    float y[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) y[c] = pooled[c] * r * (gamma ? gamma[8 * lane + c] : 1.0f);
    *reinterpret_cast<float4*>(&yS[ei][8 * lane]) = make_float4(y[0], y[1], y[2], y[3]);
    *reinterpret_cast<float4*>(&yS[ei][8 * lane + 4]) = make_float4(y[4], y[5], y[6], y[7]);
    if (cs == 0) {
      // compressed RoPE of the main entry: lanes 56..63 hold dims 448..511,
      // pairs (c, c+1) of the lane's 8 channels
      if (rope_pos && lane >= 56) {
        const int64_t pos = rope_pos[e];
#pragma unroll
        for (int c = 0; c < 8; c += 2) {
          float cz, sn;
          rope_cos_sin(pos, 4 * (lane - 56) + c / 2, cz, sn);
          rope_pair<false>(y[c], y[c + 1], cz, sn);
        }
      }
      // main-KV FP4: a group of 16 channels spans two lanes
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) amax = fmaxf(amax, fabsf(y[c]));
      amax = group_reduce<2, true>(amax);
      const uint32_t b = scale_code<FMT>(amax);
      const float sv = scale_value<FMT>(b);
      const uint32_t word = e2m1x8<FMT>(y, sv);
      *reinterpret_cast<uint32_t*>(main_codes + e * 256 + 4 * lane) = word;
      if ((lane & 1) == 0) main_scales[e * 32 + lane / 2] = (uint8_t)b;
    }
  }
  __syncthreads();

  // ---- phase 2: K steps ks0 .. ks0 + kSteps - 1 of column group `grp`.
  // A: lane (g, n) holds Y[entry n][128g + ks]; MFMA j's B: W[128g + ks][d + j];
  // its D: lane (g, n) holds K[entries 4g .. 4g+3][d + j].
  floatx4 acc[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s4 = 0; s4 < kSteps; s4 += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(&yS[n][128 * g + ks0 + s4]);
    const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int st = s4 + i;
      const wvec bv = wpre[st % kPre];
      if (st + kPre < kSteps)
        wpre[st % kPre] = *reinterpret_cast<const wvec*>(w_idx + (128 * g + ks0 + st + kPre) * 128 + d);
#pragma unroll
      for (int j = 0; j < kJ; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[j], 0, 0, 0);
    }
  }
  // partial products of the waves of each column group, summed into kS
  // (column c - 16T*cs of this split): part[wave][256 j + 64 i + lane]
  __syncthreads();  // every wave is done reading Y
#pragma unroll
  for (int j = 0; j < kJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[wave][256 * j + 64 * i + lane] = acc[j][i];
  __syncthreads();
  for (int o = threadIdx.x; o < kGroups * kJ * 256; o += 64 * kWriteWaves) {
    const int gg = o / (kJ * 256), jl = o % (kJ * 256);
    const int j = jl >> 8, i = (jl >> 6) & 3, ln = jl & 63;
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < kWpg; ++r) v += part[gg * kWpg + r][jl];
    kS[4 * (ln >> 4) + i][kCW * gg + kJ * (ln & 15) + j] = v;
  }
  __syncthreads();

  // ---- phase 3: indexer-K FP4 (E8M0, groups of 32 columns): thread ->
  // (entry, 8 consecutive columns of this split); 4 threads share a group
  if ((int)threadIdx.x < kWriteEntries * 2 * T) {
    const int ei = threadIdx.x / (2 * T), ch = threadIdx.x % (2 * T);
    const int64_t e = e0 + ei;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = kS[ei][8 * ch + j];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = group_reduce<4, true>(amax);
    const uint32_t b = scale_code_e8m0(amax);
    const uint32_t word = e2m1x8_pow2(v, e8m0_value(b));
    if (e < n_entries) {
      const int col0 = 16 * T * cs + 8 * ch;  // first column of these 8
      *reinterpret_cast<uint32_t*>(idx_codes + e * 64 + col0 / 2) = word;
      if ((ch & 3) == 0) idx_scales[e * 4 + col0 / 32] = (uint8_t)b;
    }
  }
}

int launch_cache_write(const uint16_t* latent, const uint16_t* gate, int64_t T, int m,
                       const float* gamma, float eps, const float* w_idx, int main_fmt,
                       const int64_t* rope_pos, uint8_t* main_codes, uint8_t* main_scales,
                       uint8_t* idx_codes, uint8_t* idx_scales, hipStream_t st) {
  const int64_t n = T / m;
  if (n == 0) return 0;
  const int64_t tiles = (n + kWriteEntries - 1) / kWriteEntries;
  // column tiles per workgroup: all 8 once the entry tiles fill the chip,
  // else split the columns so that about 256 workgroups run (splitting a
  // 4096-entry write over 512 workgroups measured slower: the pooling and
  // the W reads are repeated per column split)
  const int tpw = tiles >= 256 ? 8 : (tiles >= 128 ? 4 : 2);
  const dim3 grid((unsigned)tiles, 8 / tpw);
  const unsigned threads = 64 * kWriteWaves;
#define CSA2_WRITE(F, TT)                                                                              \
  cache_write_kernel<F, TT><<<grid, threads, 0, st>>>(latent, gate, n, m, gamma, eps, w_idx, rope_pos, \
                                                      main_codes, main_scales, idx_codes, idx_scales)
  if (main_fmt == 0) {
    if (tpw == 8) CSA2_WRITE(0, 8); else if (tpw == 4) CSA2_WRITE(0, 4); else CSA2_WRITE(0, 2);
  } else {
    if (tpw == 8) CSA2_WRITE(1, 8); else if (tpw == 4) CSA2_WRITE(1, 4); else CSA2_WRITE(1, 2);
  }
#undef CSA2_WRITE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ------------------------------------------------------------ decode append
// [jokeuncle.pages.dev, "两张架构图里藏着 890 字节", section 四 item 1;
// ggaaooppeenngg.github.io, "架构解析：KV Cache 压缩的极限在哪里", 3.2]: a decoder
// layer (m = 1) writes one compressed entry per generated token; a layer with
// m = 2 writes one every second token, holding the first token of each group
// until its partner arrives.  One new token per sequence per call; the entry
// goes to row len[b] of the sequence's planes (with RoPE at position len[b]
// when asked) and len[b] advances.  Two launches: the write, then the
// advance (so that no workgroup of the write reads a length already moved).
// State for m = 2 (caller-owned, zero-filled once): int32 count[B] (tokens
// held, 0 or 1), then bf16 latent[B][512] and gate[B][512] of the held token.
struct AppendState {
  int32_t* count;
  uint16_t* lat;
  uint16_t* gate;
};

static AppendState append_state(void* st, int B) {
  char* p = reinterpret_cast<char*>(st);
  const size_t c = ((size_t)B * 4 + 255) & ~(size_t)255;
  return AppendState{reinterpret_cast<int32_t*>(p), reinterpret_cast<uint16_t*>(p + c),
                     reinterpret_cast<uint16_t*>(p + c + (size_t)B * 1024)};
}

size_t append_state_bytes(int B) { return (((size_t)B * 4 + 255) & ~(size_t)255) + (size_t)B * 2048; }

// Grid (sequence, 4 column tiles), 256 threads: thread t pools and
// normalises channels 2t, 2t+1 (the cache write's operations, in its order);
// in column tile 0, threads 0..31 quantise the main entry (one 16-channel
// group each, RoPE on groups 28..31); every workgroup projects onto its 32
// indexer-K columns (one E8M0 group), 8 channel slices of 64 per column.
template <int FMT>
__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ gate, int m,
    const float* __restrict__ gamma, float eps, const float* __restrict__ w_idx, int rope,
    uint8_t* __restrict__ main_codes, uint8_t* __restrict__ main_scales,
    uint8_t* __restrict__ idx_codes, uint8_t* __restrict__ idx_scales, int64_t cap,
    const int32_t* __restrict__ len, const int32_t* __restrict__ count,
    const uint16_t* __restrict__ plat, const uint16_t* __restrict__ pgate, PageMap pm) {
  __shared__ float y[512];
  __shared__ float kv[8][33];
  __shared__ float red[4];
  __shared__ uint32_t kc[32];
  const int b = blockIdx.x, ct = blockIdx.y, t = threadIdx.x;
  const int32_t L = len[b];
  if (L < 0 || (int64_t)L >= cap) return;    // full: nothing is written (uniform)
  if (m == 2 && count[b] == 0) return;      // first token of a group: the advance holds it
  float pooled[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int64_t i = (int64_t)b * 512 + 2 * t + c;
    if (m == 1) {
      pooled[c] = bf16_bits_to_f32(latent[i]);
    } else {
      pooled[c] = pool2(bf16_bits_to_f32(pgate[i]), bf16_bits_to_f32(gate[i]), bf16_bits_to_f32(plat[i]),
                        bf16_bits_to_f32(latent[i]));
    }
  }
  float ss = wave_sum(pooled[0] * pooled[0] + pooled[1] * pooled[1]);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(ss / 512.0f + eps);
#pragma unroll
  for (int c = 0; c < 2; ++c) y[2 * t + c] = pooled[c] * r * (gamma ? gamma[2 * t + c] : 1.0f);
  __syncthreads();
  // entry L of sequence b: its own region, or its page of the pool
  const int64_t row = pm.table ? (int64_t)page_row(pm, b, L) : (int64_t)b * cap + L;
  if (ct == 0 && t < 32) {
    // main entry, channel group t (16 channels), rotated first when asked
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = y[16 * t + j];
    if (rope && t >= 28) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        float cs, sn;
        rope_cos_sin(L, 8 * (t - 28) + j / 2, cs, sn);
        rope_pair<false>(v[j], v[j + 1], cs, sn);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const uint32_t sb = scale_code<FMT>(amax);
    const float sc = scale_value<FMT>(sb);
    float v0[8], v1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v0[j] = v[j];
      v1[j] = v[8 + j];
    }
    *reinterpret_cast<uint2*>(main_codes + row * 256 + 8 * t) = make_uint2(e2m1x8<FMT>(v0, sc), e2m1x8<FMT>(v1, sc));
    main_scales[row * 32 + t] = (uint8_t)sb;
  }
  // indexer key from the unrotated entry: thread = (channel slice, column)
  {
    const int col = t & 31, sl = t >> 5;
    float wv[64];
#pragma unroll
    for (int c = 0; c < 64; ++c) wv[c] = w_idx[(64 * sl + c) * 128 + 32 * ct + col];
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) acc += y[64 * sl + c] * wv[c];
    kv[sl][col] = acc;
  }
  __syncthreads();
  if (t < 32) {
    float v = 0.f;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) v += kv[s8][t];
    float amax = fabsf(v);
    amax = group_reduce<32, true>(amax);
    const uint32_t sb = scale_code_e8m0(amax);
    kc[t] = e2m1_pow2(v, e8m0_value(sb));
    if (t == 0) idx_scales[row * 4 + ct] = (uint8_t)sb;
  }
  __syncthreads();
  if (t < 4) {
    uint32_t w = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= kc[8 * t + j] << (4 * j);
    *reinterpret_cast<uint32_t*>(idx_codes + row * 64 + 16 * ct + 4 * t) = w;
  }
}

// After the write: advance len (m = 1, or the second token of an m = 2
// group), or hold the token (first of an m = 2 group).  A full sequence is
// left as it is.  One wave per sequence.
__global__ __launch_bounds__(64) void cache_advance_kernel(
    const uint16_t* __restrict__ latent, const uint16_t* __restrict__ gate, int m, int64_t cap,
    int32_t* __restrict__ len, int32_t* __restrict__ count, uint16_t* __restrict__ plat,
    uint16_t* __restrict__ pgate) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int32_t L = len[b];
  const bool full = L < 0 || (int64_t)L >= cap;
  const int32_t c = m == 2 ? count[b] : 1;
  __syncthreads();  // every lane has read len and count before lane 0 moves them
  if (full) return;
  if (c == 0) {
    const uint4* src = reinterpret_cast<const uint4*>(latent + (int64_t)b * 512);
    const uint4* srg = reinterpret_cast<const uint4*>(gate + (int64_t)b * 512);
    reinterpret_cast<uint4*>(plat + (int64_t)b * 512)[t] = src[t];
    reinterpret_cast<uint4*>(pgate + (int64_t)b * 512)[t] = srg[t];
    if (t == 0) count[b] = 1;
  } else if (t == 0) {
    if (m == 2) count[b] = 0;
    len[b] = L + 1;
  }
}

int launch_cache_append(const uint16_t* latent, const uint16_t* gate, int B, int m, const float* gamma,
                        float eps, const float* w_idx, int main_fmt, int rope, uint8_t* main_codes,
                        uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales, int64_t cap,
                        int32_t* len, void* state, hipStream_t st, PageMap pm) {
  if (B == 0) return 0;
  AppendState s{nullptr, nullptr, nullptr};
  if (m == 2) s = append_state(state, B);
  if (main_fmt == 0)
    cache_append_kernel<0><<<dim3(B, 4), 256, 0, st>>>(latent, gate, m, gamma, eps, w_idx, rope, main_codes,
                                              main_scales, idx_codes, idx_scales, cap, len, s.count, s.lat,
                                              s.gate, pm);
  else
    cache_append_kernel<1><<<dim3(B, 4), 256, 0, st>>>(latent, gate, m, gamma, eps, w_idx, rope, main_codes,
                                              main_scales, idx_codes, idx_scales, cap, len, s.count, s.lat,
                                              s.gate, pm);
  cache_advance_kernel<<<B, 64, 0, st>>>(latent, gate, m, cap, len, s.count, s.lat, s.gate);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ======================================================================
// FP8 sliding-window ring
// ======================================================================
// Record of one window slot: 576 data bytes -- OCP E4M3 codes of dims
// 0..447 with one UE8M0 scale per 64 dims, then dims 448..511 as bf16 -- and
// 8 scale bytes (7 scales and a zero pad).  The window keeps the token's own
// RMS-normalised latent (no pooling), rotated at the token's position.

// smallest UE8M0 byte b with 448 * 2^(b-127) >= amax (0 for amax == 0):
// amax = f * 2^e with f in [0.5, 1) and 448 = 0.875 * 2^9
__device__ __forceinline__ uint32_t fp8_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0u;
  int e;
  const float f = frexpf(amax, &e);
  const int b = e + 118 + (f > 0.875f ? 1 : 0);
  return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// nearest OCP E4M3 code of v (|v| <= 448), ties to the even code; +0 for a
// zero magnitude.  With a = |v| in binade E (floored at -6, the subnormal
// exponent) the step is 2^(E-3) and code = 8 (E + 7) + n - 8 for the rounded
// multiple n; n = 16 moves to the next binade by itself, and E = -6 with
// n < 8 gives the subnormal code n.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float a = fabsf(v);
  if (a == 0.0f) return 0u;
  int e;
  (void)frexpf(a, &e);
  const int E = max(e - 1, -6);
  const int nq = (int)rintf(ldexpf(a, 3 - E));
  const uint32_t code = (uint32_t)(8 * (E + 7) + nq - 8);
  return (code != 0u && v < 0.0f) ? (code | 0x80u) : code;
}

// Grid (sequence, written token), one wave: lane t takes dims 8t..8t+7.
// Only the last min(n, W) tokens are written (earlier ones would be
// overwritten in the ring anyway).
__global__ __launch_bounds__(64) void window_write_kernel(
    const uint16_t* __restrict__ latent, int n, const float* __restrict__ gamma, float eps, int rope,
    const int64_t* __restrict__ pos0, int W, uint8_t* __restrict__ data, uint8_t* __restrict__ scales,
    int32_t* __restrict__ swa_len) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int nw = n < W ? n : W;
  const int i = n - nw + (int)blockIdx.y;
  const int64_t p0 = pos0[b];
  if (p0 < 0) return;  // not a position: the sequence is left as it is (uniform)
  const int64_t p = p0 + i;
  if (blockIdx.y == 0 && t == 0) swa_len[b] = (int32_t)(p0 + n < W ? p0 + n : W);
  const uint4 raw = reinterpret_cast<const uint4*>(latent + ((int64_t)b * n + i) * 512)[t];
  const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = bf16_bits_to_f32(wd[j] & 0xFFFFu);
    v[2 * j + 1] = bf16_bits_to_f32(wd[j] >> 16);
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) ss += v[j] * v[j];
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / 512.0f + eps);
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = v[j] * r * (gamma ? gamma[8 * t + j] : 1.0f);
  uint8_t* rec = data + ((int64_t)b * W + p % W) * 576;
  // per 64-dim group (8 lanes): the largest magnitude and its scale byte
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = group_reduce<8, true>(amax);
  const uint32_t sb = fp8_scale_code(amax);
  uint32_t sbytes[8];
#pragma unroll
  for (int gi = 0; gi < 8; ++gi) sbytes[gi] = (uint32_t)__builtin_amdgcn_readlane((int)sb, 8 * gi);  // uniform
  if (t < 56) {
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j >> 2] |= e4m3_code(ldexpf(v[j], 127 - (int)sb)) << (8 * (j & 3));
    *reinterpret_cast<uint2*>(rec + 8 * t) = make_uint2(c[0], c[1]);
  } else {
    if (rope) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        float cs, sn;
        rope_cos_sin(p, 4 * (t - 56) + j / 2, cs, sn);
        rope_pair<false>(v[j], v[j + 1], cs, sn);
      }
    }
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    *reinterpret_cast<uint4*>(rec + 448 + 16 * (t - 56)) = make_uint4(h[0], h[1], h[2], h[3]);
  }
  if (t == 0) {
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) lo |= sbytes[gi] << (8 * gi);
#pragma unroll
    for (int gi = 4; gi < 7; ++gi) hi |= sbytes[gi] << (8 * (gi - 4));
    *reinterpret_cast<uint2*>(scales + ((int64_t)b * W + p % W) * 8) = make_uint2(lo, hi);
  }
}

int launch_window_write(const uint16_t* latent, int B, int n, const float* gamma, float eps, int rope,
                        const int64_t* pos0, int W, uint8_t* data, uint8_t* scales, int32_t* swa_len,
                        hipStream_t st) {
  if (B == 0) return 0;
  const int nw = n < W ? n : W;
  window_write_kernel<<<dim3(B, nw), 64, 0, st>>>(latent, n, gamma, eps, rope, pos0, W, data, scales, swa_len);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
