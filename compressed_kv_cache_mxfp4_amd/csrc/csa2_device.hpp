// csa2_device.hpp -- device-side helpers shared by the CSA2 kernels (gfx950).
//
// FP4 cache rows are E2M1 nibbles (value 2i in the low nibble of byte i) with
// one scale byte per group [jokeuncle.pages.dev, "两张架构图里藏着 890 字节",
// section 三].  Decoding uses the gfx950 scaled-convert instructions; their
// scale operand is a power of two carried in the exponent field of an fp32,
// which is exactly an E8M0 byte shifted into place.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// E8M0 byte as the fp32 power of two the scaled converts expect (b << 23;
// b = 0 encodes 2^-127 the same way the hardware reads exponent field 0).
__device__ __forceinline__ float e8m0_operand(uint32_t b) { return __uint_as_float(b << 23); }

// Exact value of an E8M0 byte as an fp32 (0 -> 2^-127, a subnormal).
__device__ __forceinline__ float e8m0_value(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : (b == 255 ? __uint_as_float(0x7FC00000u) : __uint_as_float(b << 23));
}

// Exact value of an OCP E4M3FN byte (sign honoured), without branches (it
// sits in the inner loops, where a divergent branch per call serialises):
// exponent e >= 1 is 2^(e-7) (1 + m/8), the fp32 with the 7 low bits moved
// into place and the exponent rebiased by 120; e = 0 is m * 2^-9; 0x7F is NaN.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t mag = b & 0x7Fu;
  const float nrm = __uint_as_float((mag << 20) + (120u << 23));
  const float sub = (float)(mag & 7u) * 0x1p-9f;
  float v = mag < 8u ? sub : nrm;
  v = mag == 0x7Fu ? __uint_as_float(0x7FC00000u) : v;
  return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// Two E2M1 values of byte `sel` of `codes` -> bf16 pair, times 2^(b-127).
template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16(uint32_t codes, float e8m0_op) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, e8m0_op, SEL);
}

// Eight E2M1 values (one dword) -> bf16x8 with an E8M0 scale.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t codes, float e8m0_op) {
  bf16x2 a = fp4x2_to_bf16<0>(codes, e8m0_op);
  bf16x2 b = fp4x2_to_bf16<1>(codes, e8m0_op);
  bf16x2 c = fp4x2_to_bf16<2>(codes, e8m0_op);
  bf16x2 d = fp4x2_to_bf16<3>(codes, e8m0_op);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ------------------------------------------------------------ compressed RoPE
// [ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析", 3.2 and 7]: base
// 160000; 64 of the 512 dims carry position.  These are dims 448..511 as 32
// adjacent pairs; pair j turns by pos * 160000^(-2j/64).  The angle is kept
// in fp64 (positions reach millions, where an fp32 angle is off by tenths of
// a radian); the rotation itself is fp32.
//
// cos and sin of the compressed-RoPE angle of pair j at position pos:
// pos * 160000^(-2j/64) radians.  The angle is carried in half-turns,
// pos * theta_j / pi with theta_j / pi = 2^(-j log2(160000)/32 - log2(pi)) in
// fp64 (within 14 ulp of exact), and sincospi drops the whole turns exactly,
// so positions in the billions keep ~1e-6 rad; a general fp64 pow and a
// large-argument sincos cost several times more.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, int j, float& c, float& s) {
  const double ht = (double)pos * exp2(-(double)j * (log2(160000.0) / 32.0) - log2(3.14159265358979323846));
  double sd, cd;
  sincospi(ht, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// Turn the pair (a, b) = (x[2j], x[2j+1]) of the RoPE dims by +angle, or by
// -angle when INV.
template <bool INV>
__device__ __forceinline__ void rope_pair(float& a, float& b, float c, float s) {
  const float sn = INV ? -s : s;
  const float x = a * c - b * sn;
  const float y = a * sn + b * c;
  a = x;
  b = y;
}

// ------------------------------------------------------------ wave helpers

// Max and sum over lanes l, l^16, l^32, l^48 (one value per 16-lane row)
// without an LDS round trip: v_permlane16_swap exchanges the odd and even
// rows, v_permlane32_swap the two halves.  Each swap leaves the lane's own
// value and its partner's in the two results, the same pair in every lane of
// the pair, so the sums are bitwise equal across the four lanes.
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A lane's value from another lane of its 16-lane row, by a DPP control
// (every lane reads; row and bank masks full).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)__float_as_uint(v), CTRL, 0xf, 0xf, true));
}

// Sum (MAX = false) or maximum over each aligned group of N lanes, N = 2 ..
// 64, without an LDS round trip.  Partners 1 and 2 lanes away come from DPP
// quad permutes; then, once each quad (half-row) holds one value, the row
// half-mirror (row mirror) reads a lane of the other quad (half-row), which
// holds what the partner 4 (8) lanes away holds; rows 16 and 32 lanes away
// come from v_permlane16_swap and v_permlane32_swap.  Each step combines the
// lane's value with the value its xor partner holds, so the results equal
// those of an xor butterfly bit for bit (the combining operations are
// commutative), and every lane of a group ends with the same value.
template <int N, bool MAX>
__device__ __forceinline__ float group_reduce(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (N >= 2) v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  if constexpr (N >= 16) v = op(v, dpp_f<0x140>(v));  // row_mirror
  if constexpr (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if constexpr (N >= 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_reduce<64, false>(v); }

__device__ __forceinline__ float wave_max(float v) { return group_reduce<64, true>(v); }

// Eight OCP E4M3 bytes (two dwords, byte i = element i) -> bf16x8, each
// times the power of two of an E8M0 operand (exact: E4M3 values scaled by a
// power of two fit in bf16 for every scale a window record uses).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi, float e8m0_op) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, e8m0_op, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, e8m0_op, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, e8m0_op, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, e8m0_op, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values -> bf16 pair (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

// Two fp32 values -> fp16 pair, round to nearest even: one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

}  // namespace csa2
