// attn.hip -- CSA2 core sparse attention for one decode query per sequence
// (gfx950).
//
// [syt-nju.github.io, "为什么读输入只激活 8B", section CSA2 / Figure 4]: the
// selected main-KV entries are concatenated with the layer's sliding-window
// entries and attended by the layer's own query; [same page, "FP4 主 KV 缓存"]
// FP4 is a storage format and rows are dequantised before the products.  Each
// row is one 512-d latent used as both key and value (one KV head shared by
// the query heads).  [jokeuncle.pages.dev, "两张架构图里藏着 890 字节", 顺便算清
// 另外三笔账]: 512 selected + 128 window rows per query.
//
// Split-rows design (flash decoding).  The row slots of a sequence (top-k
// entries, then window entries) are cut into chunks of 16*WAVES slots (128 or
// 160); one workgroup takes one (sequence, 16 heads, chunk), so a decode call
// with 16 sequences, 64 heads and 512 + 128 rows runs 256-320 workgroups
// rather than 64.  Each workgroup leaves a partial output (normalised by its
// own sum, stored as fp16 scaled by a power of two) with its max and sum; the
// last workgroup of a (sequence, head group) to finish merges the chunks
// exactly, in a fixed order.
//  * Q.R^T: wave w takes rows 16w..16w+15 of the chunk.  Lane (g, m) holds the
//    code bytes of row m for dims 64g..64g+63 and 256+64g..256+64g+63 and
//    their 8 scale bytes, and dequantises them straight into the A operand of
//    v_mfma_f32_16x16x32_bf16: K step ks covers dims 64g+8ks (ks < 8) or
//    256+64g+8(ks-8) in lane group g.  The query fragments (B operand) come
//    from one LDS copy of the 16 queries with the same permutation (loading
//    them per wave from global memory would move 8x the bytes through the
//    CU's vector-memory path).  Every row is dequantised exactly once; the
//    bf16 values stay in registers until their half of R is staged.
//  * P.R: each 256-dim half of R lives in LDS in turn (67 KB at 8 waves, so
//    two workgroups share a CU); of the half's sixteen 16-dim tiles wave w
//    takes tiles w and w+WAVES (when below 16) for the 16 heads.  P comes from LDS; the row-major R tile is read column-wise
//    with the gfx950 transpose read (ds_read_b64_tr_b16): within a 16-lane
//    group, source lane a+4j points at R[r0+j][d0+4a] and lane n receives
//    R[r0..r0+3][d0+n], i.e. four K slots of the MFMA B operand.
#include <type_traits>

#include "csa2.h"
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kChunk = 128;            // row slots per workgroup at most 8 waves (sizes the workspace)
constexpr int kHLd = 256;              // R half-row stride in bf16 (no pad: rows are swizzled)
constexpr int kQLd = 520;              // query row stride in bf16 (512 + pad)
// s_getreg operand for HW_REG_XCC_ID (register 20, bits 3:0): the XCD a wave runs on
constexpr int kHwRegXccId = (3 << 11) | 20;
// completion counters: one per (sequence, head group), in a fixed region at
// the start of the workspace so that no call shape ever overlays them
constexpr int kMaxAttnGroups = 65536;

typedef short shortx4 __attribute__((ext_vector_type(4)));

// MFMA operand type of the split kernel: bf16, or fp16 for E4M3-scaled main
// rows (an E2M1 value times an E4M3 scale is exact in fp16 as in bf16, and
// fp16 lets the scale's significand be applied two values per instruction).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool F16>
struct OpT {
  using v8 = bf16x8;
};
template <>
struct OpT<true> {
  using v8 = f16x8;
};

template <bool F16>
__device__ __forceinline__ floatx4 mfma16(typename OpT<F16>::v8 a, typename OpT<F16>::v8 b, floatx4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Staged R half-rows are 512 B; 16-byte unit u of row r sits at unit
// u ^ rswz(r).  gfx950's LDS has 64 banks of 4 B (256 B); measured there,
// a transposed 8-byte read serves 32 lanes per cycle and a 16-byte write
// 16.  The transposed reads of P.R give the 32 lanes of a half-wave units
// 2t and 2t+1 of rows {0..3, 8..11} (or {4..7, 12..15}) + a multiple of 16:
// bits 1-3 of rswz (r & 3 and bit 3 of r) send those 8 rows' 32-byte pairs
// to 8 distinct 32-byte bank slots (2 cycles per read, against 4 with a
// 2-way conflict).  The staging writes give the 16 lanes of a quarter-wave
// unit 8g + ks of 16 consecutive rows; bit 0 (bit 2 of r) makes the 16
// swizzles distinct, so those are conflict-free too.
__device__ __forceinline__ int rswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3); }

// bf16 index of 16-byte unit u of staged row r.
__device__ __forceinline__ int runit(int r, int u) { return r * kHLd + ((u ^ rswz(r)) << 3); }

// Arrival of a workgroup at its group's completion counter, after it has
// stored its partial; true in every thread of the workgroup that arrives last
// (n arrivals per group), which then reads the others' partials.  Why a
// relaxed counter suffices on gfx950, without agent-scope fences:
//  * the grids give every workgroup of a group an id congruent mod 8, and
//    gfx950 dispatches workgroup i of a launch to XCD i mod 8, so a group's
//    writers and its merger share one L2 (each partial records the XCD its
//    writer ran on, and the merge turns its output into NaN if any differs
//    from its own -- never observed);
//  * the vector L1 is write-through, and each wave waits for its stores to be
//    acknowledged (s_waitcnt 0) before the barrier that precedes the counter
//    update, so every partial is in that L2 before the counter moves;
//  * the merger's L1 holds no stale copy: no other workgroup reads a group's
//    partials, they occupy cache lines of their own (1 KB rows and 16-B
//    records in runs of whole 256-B multiples), and the L1 is invalidated at
//    kernel start.
// The agent-scope release/acquire pair the HIP memory model asks for when
// writers may sit on other XCDs (an L2 write-back per arriving workgroup and
// an L2 invalidate per merge) took the decode call at batch 16 from 12.2 to
// 18.5 us.  The last arrival resets the counter, so it is zero again when the
// kernel ends.
__device__ __forceinline__ bool arrive_last(uint32_t* c, uint32_t n, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = old == n - 1u;
    if (old == n - 1u) *c = 0u;  // ready for the next call
  }
  __syncthreads();
  return *flag != 0;
}

// WAVES waves take 16 rows each: a chunk of 16*WAVES row slots.  With more
// than 8 waves one workgroup fills a CU, and the query tile gets a region of
// its own so that each wave can stage its rows as soon as its logits are
// done; with 8 waves (two workgroups per CU) the query tile borrows R.
template <int WAVES>
struct AttnSmem {
  static constexpr int kRows = 16 * WAVES;
  // P plane row (one head) in bf16: kRows / 2 slots + 4 pad (8-byte reads of
  // 16 heads then hit 16 distinct bank pairs)
  static constexpr int kPP = kRows / 2 + 4;
  static constexpr bool kQOwn = WAVES > 8;
  uint16_t R[kRows * kHLd];
  uint16_t Qown[kQOwn ? 16 * kQLd : 8];
  // P as two planes of 8-byte halves, plane 0 (row slots 8u..8u+3 of each
  // 8-slot unit) then plane 1 (8u+4..8u+7): an MFMA operand is two 8-byte
  // reads, which gfx950's LDS serves in 8 cycles against 16 for one 16-byte
  // read of 64 distinct units (measured)
  uint16_t P[2 * 16 * kPP];
  __align__(16) float red_m[WAVES][16];
  __align__(16) float red_l[WAVES][16];
  float red_v[WAVES];  // per-wave bound of |dequantised value| (partial scaling)
  int qk[16];          // fp16 operands: the query of head h is staged times 2^-qk[h]
  uint2 e4lut[256];    // fp16 operands: (power of two, significand pair) of each E4M3 scale byte
  int last;  // this workgroup merges its (sequence, head group)
};

// Compressed RoPE of 8 consecutive bf16 dims starting at dim d0 (a multiple
// of 8, >= 448): the 4 pairs turn by +angle at `pos`; the result is rounded
// back to bf16 (nearest-even).
__device__ __forceinline__ uint4 rope_bf16x8(uint4 v, int d0, int64_t pos) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = bf16_bits_to_f32(w[i] & 0xFFFFu), b = bf16_bits_to_f32(w[i] >> 16);
    float c, sn;
    rope_cos_sin(pos, (d0 - 448) / 2 + i, c, sn);
    rope_pair<false>(a, b, c, sn);
    w[i] = pack_bf16x2(a, b);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Eight E2M1 values of one code dword -> bf16x8 (exact).  E4M3 scales: the
// scaled convert honours only the exponent of its fp32 scale, so it is given
// the scale's power of two and the products are finished in fp32 by the
// scale's significand (1 + m/8, or the subnormal code's m).  An E2M1 value
// (at most 2 significant bits) times an E4M3 scale (at most 4) has at most 5
// significant bits, so each fp32 product is a bf16 value and its upper half
// is the bf16 encoding: the pairs are packed by a byte permute, no rounding.
template <int FMT>
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, uint32_t sbyte) {
  if (FMT == 0) {
    return fp4x8_to_bf16(codes, e8m0_operand(sbyte));
  } else {
    const float s = e4m3_value(sbyte);  // a normal fp32 (>= 2^-9) or NaN
    // |s| = 2^E * sig with sig in [1, 2): the convert takes the power of two
    // 2^E; sig carries the sign (and NaN for the NaN codes)
    const uint32_t su = __float_as_uint(s);
    const float sig = s != s ? s : __uint_as_float((su & 0x807FFFFFu) | 0x3F800000u);
    const float sa = __uint_as_float(su & 0x7F800000u);
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sa, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sa, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sa, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, sa, 3);
    auto hi2 = [](float a, float b) {  // bf16(b) << 16 | bf16(a), both exact
      return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
    };
    uint4 u;
    u.x = hi2(p0[0] * sig, p0[1] * sig);
    u.y = hi2(p1[0] * sig, p1[1] * sig);
    u.z = hi2(p2[0] * sig, p2[1] * sig);
    u.w = hi2(p3[0] * sig, p3[1] * sig);
    return __builtin_bit_cast(bf16x8, u);
  }
}

// Eight E2M1 values of one code dword with an E4M3 scale byte -> fp16x8
// (exact): the scaled convert takes the scale's power of two, v_pk_mul_f16
// its significand, two values per instruction.
struct E4m3F16 {
  float pow2;  // the scale's power of two (the scaled convert's operand)
  f16x2 sig;   // its significand (sign, NaN) twice, for v_pk_mul_f16
};

__device__ __forceinline__ E4m3F16 e4m3_f16_scale(uint32_t sbyte) {
  const float s = e4m3_value(sbyte);  // a normal fp32 (>= 2^-9) or NaN
  const uint32_t su = __float_as_uint(s);
  const _Float16 h = (_Float16)(s != s ? s : __uint_as_float((su & 0x807FFFFFu) | 0x3F800000u));
  return E4m3F16{__uint_as_float(su & 0x7F800000u), f16x2{h, h}};
}

__device__ __forceinline__ f16x8 dequant8_f16(uint32_t codes, const E4m3F16& sc) {
  const float sa = sc.pow2;
  const f16x2 sg = sc.sig;
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sa, 0) * sg;
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sa, 1) * sg;
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sa, 2) * sg;
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sa, 3) * sg;
  f16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// bf16x8 (8 dims of one query head) -> fp16x8 times 2^-k (exact for
// magnitudes from 2^-14; smaller ones are rounded to fp16's subnormal grid).
__device__ __forceinline__ uint4 bf16x8_to_f16_scaled(uint4 v, int k) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // times 2^-k exactly (v_ldexp_f32: any k a bf16 head needs)
    o[i] = pack_f16x2(ldexpf(bf16_bits_to_f32(wd[i] & 0xFFFFu), -k), ldexpf(bf16_bits_to_f32(wd[i] >> 16), -k));
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Exponent shift of one query head for fp16 operands: the k with
// 2^14 <= max|q| * 2^-k < 2^15 (the wave holds one head: 64 lanes x 8 dims),
// so the largest component sits at the top of fp16's range and every
// component above 2^-28 of it stays a normal fp16, holding its 8 bf16
// significant bits exactly.  k is negative for heads below 2^14 (down to
// -147 for bf16's smallest subnormal) and at most 113 (bf16's largest value).
__device__ __forceinline__ int head_shift_f16(uint4 v) {
  const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(wd[i] & 0xFFFFu)), fabsf(bf16_bits_to_f32(wd[i] >> 16))));
  m = wave_max(m);  // DPP and row swaps, no LDS
  if (!(m > 0.0f) || !(m < INFINITY)) return 0;  // zero, inf or NaN: no shift
  int e;
  (void)frexpf(m, &e);  // 2^(e-1) <= m < 2^e
  return e - 15;
}

struct RowFetch {
  uint4 c[4];   // code bytes: c[0..1] dims 64g..64g+63, c[2..3] dims 256+64g..256+64g+63
  uint32_t s[2];  // scale bytes: s[0] groups 4g..4g+3, s[1] groups 16+4g..16+4g+3
  uint32_t ok;  // row exists and is visible
  // FP8 window record (lane group g): c[0..3] E4M3 dims 64g..64g+63,
  // x[0..2] E4M3 dims 256+48g..256+48g+47, x[3..4] bf16 dims 448+16g..+15,
  // s[0..1] the record's 8 UE8M0 bytes (byte i: dims 64i..64i+63)
  uint4 x[5];
  uint32_t win;  // the row is an FP8 window record
};

struct RowSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  uint32_t ok;
  uint32_t win;
};

// FP8 window record: 576 data bytes (E4M3 dims 0..447, bf16 dims 448..511)
// and 8 scale bytes per slot.
constexpr int kWinDataB = 576;
constexpr int kWinScaleB = 8;

// Where row slot `slot` of sequence b lives (selected entry or window entry);
// `p` is the already-loaded index-list entry for slots below k.  Window
// entries take slots kw.. (kw = k, or k rounded up to 16 for FP8 records, so
// that no wave mixes the two row layouts: a wave's query fragments follow
// one layout); slots k..kw-1 are empty.
template <bool WF8>
__device__ __forceinline__ RowSrc locate_row(int slot, int32_t p, int nslots, int b, int k, int kw,
                                             int64_t L, int SL, int64_t seq_stride, int64_t swa_stride,
                                             const uint8_t* __restrict__ main_codes,
                                             const uint8_t* __restrict__ main_scales,
                                             const uint8_t* __restrict__ swa_codes,
                                             const uint8_t* __restrict__ swa_scales) {
  RowSrc r{nullptr, nullptr, 0u, 0u};
  if (slot < k) {
    if (p >= 0 && (int64_t)p < L) {
      r.codes = main_codes + ((int64_t)b * seq_stride + p) * 256;
      r.scales = main_scales + ((int64_t)b * seq_stride + p) * 32;
      r.ok = 1u;
    }
  } else if (slot >= kw && slot < nslots) {
    const int rr = slot - kw;
    if (rr < SL) {
      const int64_t wr = (int64_t)b * swa_stride + rr;
      r.codes = swa_codes + wr * (WF8 ? kWinDataB : 256);
      r.scales = swa_scales + wr * (WF8 ? kWinScaleB : 32);
      r.ok = 1u;
      r.win = WF8 ? 1u : 0u;
    }
  }
  return r;
}

__device__ __forceinline__ void fetch_row(RowFetch& f, const RowSrc& r, int g) {
  if (r.ok) {
    const uint4* lo = reinterpret_cast<const uint4*>(r.codes + 32 * g);
    const uint4* hi = reinterpret_cast<const uint4*>(r.codes + 128 + 32 * g);
    f.c[0] = lo[0];
    f.c[1] = lo[1];
    f.c[2] = hi[0];
    f.c[3] = hi[1];
    f.s[0] = *reinterpret_cast<const uint32_t*>(r.scales + 4 * g);
    f.s[1] = *reinterpret_cast<const uint32_t*>(r.scales + 16 + 4 * g);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.c[j] = make_uint4(0u, 0u, 0u, 0u);
    f.s[0] = f.s[1] = 0u;
  }
  f.ok = r.ok;
}

// FP8 window record: the lane's slice as in RowFetch (an invisible row reads
// as zeros).
__device__ __forceinline__ void fetch_row_w8(RowFetch& f, const RowSrc& r, int g) {
  if (r.ok && r.win) {
    const uint4* lo = reinterpret_cast<const uint4*>(r.codes + 64 * g);
    const uint4* hi = reinterpret_cast<const uint4*>(r.codes + 256 + 48 * g);
    const uint4* rp = reinterpret_cast<const uint4*>(r.codes + 448 + 32 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.c[j] = lo[j];
#pragma unroll
    for (int j = 0; j < 3; ++j) f.x[j] = hi[j];
    f.x[3] = rp[0];
    f.x[4] = rp[1];
    const uint2 sc = *reinterpret_cast<const uint2*>(r.scales);
    f.s[0] = sc.x;
    f.s[1] = sc.y;
  } else if (r.ok) {
    const uint4* lo = reinterpret_cast<const uint4*>(r.codes + 32 * g);
    const uint4* hi = reinterpret_cast<const uint4*>(r.codes + 128 + 32 * g);
    f.c[0] = lo[0];
    f.c[1] = lo[1];
    f.c[2] = hi[0];
    f.c[3] = hi[1];
    f.s[0] = *reinterpret_cast<const uint32_t*>(r.scales + 4 * g);
    f.s[1] = *reinterpret_cast<const uint32_t*>(r.scales + 16 + 4 * g);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.c[j] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 5; ++j) f.x[j] = make_uint4(0u, 0u, 0u, 0u);
    f.s[0] = f.s[1] = 0u;
  }
  f.ok = r.ok;
  f.win = r.ok & r.win;
}

// Dims of K step ks in lane group g for an FP8 window record: 64g+8ks
// (ks < 8), 256+48g+8(ks-8) (ks 8..13), 448+16g+8(ks-14) (ks 14, 15).
__device__ __forceinline__ int step_dim_w8(int ks, int g) {
  return ks < 8 ? 64 * g + 8 * ks : (ks < 14 ? 256 + 48 * g + 8 * (ks - 8) : 448 + 16 * g + 8 * (ks - 14));
}

// K step ks of a lane's FP8 window slice as bf16x8 (exact).
__device__ __forceinline__ bf16x8 row_step_w8(const RowFetch& f, int ks, int g) {
  if (ks >= 14) return __builtin_bit_cast(bf16x8, f.x[3 + (ks - 14)]);
  const uint4 u = ks < 8 ? f.c[ks >> 1] : f.x[(ks - 8) >> 1];
  const uint32_t lo = (ks & 1) ? u.z : u.x, hi = (ks & 1) ? u.w : u.y;
  const int grp = step_dim_w8(ks, g) >> 6;
  const uint32_t sb = (f.s[grp >> 2] >> (8 * (grp & 3))) & 0xFFu;
  return fp8x8_to_bf16(lo, hi, e8m0_operand(sb));
}

// Dims of K step ks in lane group g: 64g+8ks (ks < 8), 256+64g+8(ks-8).
__device__ __forceinline__ int step_dim(int ks, int g) {
  return (ks < 8 ? 0 : 256) + 64 * g + 8 * (ks & 7);
}

// Dequantise K step ks of one lane's row slice.
template <int FMT>
__device__ __forceinline__ bf16x8 row_step(const RowFetch& f, int ks) {
  const uint4 c4 = f.c[ks >> 2];
  const uint32_t cwd = (ks & 3) == 0 ? c4.x : ((ks & 3) == 1 ? c4.y : ((ks & 3) == 2 ? c4.z : c4.w));
  const uint32_t sbyte = (f.s[ks >> 3] >> (8 * ((ks >> 1) & 3))) & 0xFFu;
  return dequant8<FMT>(cwd, sbyte);
}

// The same step as fp16 (E4M3 scales); K steps 2j and 2j+1 share scale
// byte j, whose decoded form the caller reads once from the workgroup's
// 256-entry table (row_scale_byte gives the byte).
__device__ __forceinline__ uint32_t row_scale_byte(const RowFetch& f, int ks) {
  return (f.s[ks >> 3] >> (8 * ((ks >> 1) & 3))) & 0xFFu;
}

__device__ __forceinline__ f16x8 row_step_f16(const RowFetch& f, int ks, const E4m3F16& sc) {
  const uint4 c4 = f.c[ks >> 2];
  const uint32_t cwd = (ks & 3) == 0 ? c4.x : ((ks & 3) == 1 ? c4.y : ((ks & 3) == 2 ? c4.z : c4.w));
  return dequant8_f16(cwd, sc);
}

// A operand of P.R K step kk (32 row slots): head n, slots 32kk + 8g .. +7,
// one 8-byte read from each P plane.
template <int WAVES, bool F16>
__device__ __forceinline__ typename OpT<F16>::v8 p_operand(const AttnSmem<WAVES>& sm, int kk, int g, int n) {
  constexpr int PP = AttnSmem<WAVES>::kPP;
  const int e = n * PP + 4 * (4 * kk + g);
  const uint2 lo = *reinterpret_cast<const uint2*>(&sm.P[e]);
  const uint2 hi = *reinterpret_cast<const uint2*>(&sm.P[16 * PP + e]);
  return __builtin_bit_cast(typename OpT<F16>::v8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// O^T(the wave's 16-dim tiles of one R half x 16 heads) += R_half^T . P^T
// (lane (g, n) accumulates head n, dims 4g..4g+3 of each tile).  Wave w
// takes tiles w and w + WAVES (16 tiles per half); K steps of 32 rows.  With
// one workgroup per CU the caller reads the P operands pa once for both
// halves; at 8 waves, where registers are scarcer, each batch reads its own.
// The LDS reads of KB K steps are issued before their products (all of them
// with one workgroup per CU; two at a time at 8 waves), so a wave does not
// wait for LDS once per K step.  A wave without a second tile reads and
// multiplies its first tile twice and drops O[1].
template <int WAVES, bool F16>
__device__ __forceinline__ void pv_half(const AttnSmem<WAVES>& sm, int w, int g, int n,
                                        const typename OpT<F16>::v8 (&pa)[AttnSmem<WAVES>::kRows / 32],
                                        floatx4 (&O)[2]) {
  constexpr int NK = AttnSmem<WAVES>::kRows / 32;
  constexpr int KB = AttnSmem<WAVES>::kQOwn ? NK : 2;
  static_assert(NK % KB == 0, "K steps must split into whole batches");
  using V8 = typename OpT<F16>::v8;
  const int ta = n & 3, tj = n >> 2;
  const int t1 = w + WAVES < 16 ? w + WAVES : w;
#pragma unroll
  for (int k0 = 0; k0 < NK; k0 += KB) {
    shortx4 lo[2][KB], hi[2][KB];
    V8 pb[KB];
    if constexpr (!AttnSmem<WAVES>::kQOwn) {
#pragma unroll
      for (int j = 0; j < KB; ++j) pb[j] = p_operand<WAVES, F16>(sm, k0 + j, g, n);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // 8 bytes at dims 16*tile + 4*ta: unit 2*tile + ta/2, half ta&1
        const int u = 2 * (nt ? t1 : w) + (ta >> 1), hb = 4 * (ta & 1);
        const int r0 = 32 * (k0 + j) + 8 * g + tj;
        lo[nt][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(&sm.R[runit(r0, u) + hb]));
        hi[nt][j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)(&sm.R[runit(r0 + 4, u) + hb]));
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int j = 0; j < KB; ++j) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        shortx8 bv;
        bv[0] = lo[nt][j][0]; bv[1] = lo[nt][j][1]; bv[2] = lo[nt][j][2]; bv[3] = lo[nt][j][3];
        bv[4] = hi[nt][j][0]; bv[5] = hi[nt][j][1]; bv[6] = hi[nt][j][2]; bv[7] = hi[nt][j][3];
        // O^T tile (16 dims x 16 heads) += R^T . P^T: the same operand registers
        // with A and B swapped, so a lane ends with 4 consecutive dims of one head
        O[nt] = mfma16<F16>(__builtin_bit_cast(V8, bv), AttnSmem<WAVES>::kQOwn ? pa[k0 + j] : pb[j], O[nt]);
      }
    }
  }
}

// The last workgroup of a group merges the S chunk partials of sequence b:
// thread tid takes head h0 + (tid >> 5), dims 16*(tid & 31) .. +15, so 512
// threads merge 16 heads and 256 threads 8.  Partials are fp16 of (output / sum) * 2^-e with
// (max, sum, XCD, e) beside them; a partial written on another XCD turns the
// output into NaN (its bytes might not be visible in this XCD's L2).
// Inverse-RoPE factors of one merging thread: its dims 16*d16 .. +15 are
// pairs 8*(d16-28) .. +7 when d16 >= 28.  They depend on the query position
// and the dims, not on the head, so a thread that merges several head
// groups computes them (in fp64) once.
struct MergeRope {
  float c[8], s[8];
};

__device__ __forceinline__ MergeRope merge_rope(int64_t pos, int d16) {
  MergeRope r;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (d16 >= 28) {
      rope_cos_sin(pos, 8 * (d16 - 28) + i, r.c[i], r.s[i]);
    } else {
      r.c[i] = 1.0f;
      r.s[i] = 0.0f;
    }
  }
  return r;
}

// One round of a merge: the records and partial slices of up to four
// splits s0 .. s0+3 for one thread (head bh, dims 16*d16 .. +15).
struct MergeIn {
  float4 e[4];
  uint4 v[4][2];
};

__device__ __forceinline__ void merge_load(MergeIn& in, const float4* __restrict__ mlp,
                                           const uint4* __restrict__ src, int s0, int S, uint32_t my_xcc) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (s0 + u < S) {
      in.e[u] = mlp[s0 + u];
      in.v[u][0] = src[(s0 + u) * 64];
      in.v[u][1] = src[(s0 + u) * 64 + 1];
    } else {
      in.e[u] = make_float4(-INFINITY, 0.f, __uint_as_float(my_xcc), 0.f);
      in.v[u][0] = in.v[u][1] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// Running state of one thread's merge (splits folded in with a running maximum).
struct MergeAcc {
  float acc[16];
  float Mx, Lsum;
  bool same_xcd;
};

__device__ __forceinline__ void merge_begin(MergeAcc& A) {
#pragma unroll
  for (int j = 0; j < 16; ++j) A.acc[j] = 0.f;
  A.Mx = -INFINITY;
  A.Lsum = 0.f;
  A.same_xcd = true;
}

__device__ __forceinline__ void merge_fold(MergeAcc& A, const MergeIn& in, uint32_t my_xcc) {
  float mg = A.Mx;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    mg = fmaxf(mg, in.e[u].x);
    A.same_xcd &= __float_as_uint(in.e[u].z) == my_xcc;
  }
  if (mg == -INFINITY) return;  // nothing visible so far
  const float rs = A.Mx == -INFINITY ? 0.0f : __expf(A.Mx - mg);
  A.Lsum *= rs;
#pragma unroll
  for (int j = 0; j < 16; ++j) A.acc[j] *= rs;
  A.Mx = mg;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    // a chunk with no visible row has max -inf and a zero partial
    const float wl = in.e[u].x == -INFINITY ? 0.0f : __expf(in.e[u].x - A.Mx) * in.e[u].y;
    A.Lsum += wl;
    const float wgt = ldexpf(wl, __float_as_int(in.e[u].w));  // undo the partial's 2^-e
    const uint32_t hw[8] = {in.v[u][0].x, in.v[u][0].y, in.v[u][0].z, in.v[u][0].w,
                            in.v[u][1].x, in.v[u][1].y, in.v[u][1].z, in.v[u][1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      A.acc[2 * j] += wgt * (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[j] & 0xFFFFu));
      A.acc[2 * j + 1] += wgt * (float)__builtin_bit_cast(_Float16, (uint16_t)(hw[j] >> 16));
    }
  }
}

template <bool ROPE>
__device__ __forceinline__ void merge_store(MergeAcc& A, int64_t bh, int d16, uint16_t* __restrict__ out,
                                            float* __restrict__ lse, const MergeRope& rope) {
  float inv = A.Lsum > 0.f ? 1.0f / A.Lsum : 0.0f;
  if (!A.same_xcd) inv = __uint_as_float(0x7FC00000u);  // never expected: make it loud
  if (ROPE && d16 >= 28) {
    // output inverse RoPE: dims 16*d16 .. +15 are pairs 8*(d16-28) .. +7
#pragma unroll
    for (int i = 0; i < 8; ++i) rope_pair<true>(A.acc[2 * i], A.acc[2 * i + 1], rope.c[i], rope.s[i]);
  }
  uint32_t o8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o8[j] = pack_bf16x2(A.acc[2 * j] * inv, A.acc[2 * j + 1] * inv);
  uint4* op = reinterpret_cast<uint4*>(out + bh * 512 + 16 * d16);
  op[0] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
  op[1] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
  if (lse && d16 == 0) lse[bh] = !A.same_xcd ? inv : (A.Lsum > 0.f ? A.Mx + logf(A.Lsum) : -INFINITY);
}

template <bool ROPE>
__device__ __forceinline__ void merge_splits(int b, int h0, int H, int S, const float4* __restrict__ ml,
                                             const uint16_t* __restrict__ part, uint16_t* __restrict__ out,
                                             float* __restrict__ lse, uint32_t my_xcc, int tid,
                                             const MergeRope& rope) {
  // thread: head hh, dims 16*d16 .. +15.  Splits are merged four at a time
  // with a running maximum (one round of loads per four splits).
  const int hh = tid >> 5, d16 = tid & 31;
  const int64_t bh = (int64_t)b * H + h0 + hh;
  const float4* mlp = ml + bh * S;
  const uint4* src = reinterpret_cast<const uint4*>(part + bh * S * 512 + 16 * d16);
  MergeAcc A;
  merge_begin(A);
  for (int s0 = 0; s0 < S; s0 += 4) {
    MergeIn in;
    merge_load(in, mlp, src, s0, S, my_xcc);
    merge_fold(A, in, my_xcc);
  }
  merge_store<ROPE>(A, bh, d16, out, lse, rope);
}

// All H heads of sequence b by 512 threads, 16 heads per round, when there
// are at most four splits: the loads of round r+1 are issued before round r
// is folded, so the rounds cost one memory round trip between them rather
// than one each.
template <bool ROPE>
__device__ __forceinline__ void merge_all_heads(int b, int H, int S, const float4* __restrict__ ml,
                                                const uint16_t* __restrict__ part, uint16_t* __restrict__ out,
                                                float* __restrict__ lse, uint32_t my_xcc, int tid,
                                                const MergeRope& rope) {
  const int hh = tid >> 5, d16 = tid & 31;
  auto load_round = [&](MergeIn& in, int r) {
    const int64_t bh = (int64_t)b * H + 16 * r + hh;
    merge_load(in, ml + bh * S, reinterpret_cast<const uint4*>(part + bh * S * 512 + 16 * d16), 0, S, my_xcc);
  };
  auto finish_round = [&](const MergeIn& in, int r) {
    MergeAcc A;
    merge_begin(A);
    merge_fold(A, in, my_xcc);
    merge_store<ROPE>(A, (int64_t)b * H + 16 * r + hh, d16, out, lse, rope);
  };
  const int R = H >> 4;
  MergeIn in0, in1;
  load_round(in0, 0);
  for (int r = 0; r < R; r += 2) {
    if (r + 1 < R) load_round(in1, r + 1);
    finish_round(in0, r);
    if (r + 1 < R) {
      if (r + 2 < R) load_round(in0, r + 2);
      finish_round(in1, r + 1);
    }
  }
}

// One (sequence, 16 heads, chunk of 16*WAVES row slots).  Grid: XCD-aware
// linear order in which the head groups of one (sequence, chunk) share an XCD
// (and its L2 copy of the chunk's rows).  Writes part[(b*H+h)*S + s][512]
// (fp32, relative to the chunk max) and ml[(b*H+h)*S + s] = (max, sum).
template <int FMT, int WAVES, bool WF8>
__global__ __launch_bounds__(64 * WAVES, WAVES <= 8 ? 4 : 1) void attn_split_kernel(
    const uint16_t* __restrict__ q, int H, const uint8_t* __restrict__ main_codes,
    const uint8_t* __restrict__ main_scales, int64_t cap, const int32_t* __restrict__ len,
    const int32_t* __restrict__ topk, int k, const uint8_t* __restrict__ swa_codes,
    const uint8_t* __restrict__ swa_scales, int64_t swa_stride, int swa_cap,
    const int32_t* __restrict__ swa_len, float sm_scale, const int64_t* __restrict__ q_pos, int B, int S,
    uint16_t* __restrict__ part, float4* __restrict__ ml, uint32_t* __restrict__ cnt,
    uint16_t* __restrict__ out, float* __restrict__ lse, int seq_units, int64_t seq_stride, int qps) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  using Smem = AttnSmem<WAVES>;
  constexpr int kRows = Smem::kRows, kPP = Smem::kPP, kThreads = 64 * WAVES;
  // fp16 operands for E4M3-scaled main rows (FP8 window records stay bf16)
  constexpr bool F16 = FMT == 1 && !WF8;
  using V8 = typename OpT<F16>::v8;
  static_assert(Smem::kQOwn || 16 * kQLd <= kRows * kHLd, "query tile must fit in the R buffer");
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  // every kernel argument in SGPRs up front: one batch of argument loads and
  // one wait, instead of a load and a wait in each branch that first uses one
  asm volatile("" ::"s"(q), "s"(main_codes), "s"(main_scales), "s"(len), "s"(topk), "s"(swa_codes),
               "s"(swa_scales), "s"(swa_len), "s"(part), "s"(ml), "s"(cnt), "s"(out), "s"(lse),
               "s"(H), "s"(cap), "s"(k), "s"(swa_stride), "s"(swa_cap), "s"(sm_scale), "s"(B), "s"(S),
               "s"(seq_units), "s"(q_pos), "s"(seq_stride), "s"(qps));
  const int HG = H >> 4;
  // Placement unit: a sequence (all its head groups and chunks) when B >= 8,
  // otherwise one (sequence, head group).  A unit's workgroups get ids
  // congruent mod 8, i.e. one XCD: its L2 then holds the rows shared by the
  // head groups and every partial the merge reads.
  const int id = blockIdx.x;
  const int xcd = id & 7, r8 = id >> 3;
  const int per_unit = seq_units ? HG * S : S;
  const int unit = (r8 / per_unit) * 8 + xcd, within = r8 % per_unit;
  // Padding workgroups (unit past the end) load from unit 0's addresses and
  // leave after issuing their loads: every load below is independent, and
  // none of them waits for another or for an early exit.
  const bool valid = unit < (seq_units ? B : B * HG);  // workgroup-uniform
  const int gi = !valid ? 0 : (seq_units ? unit * HG + within / S : unit);  // (sequence, head group)
  const int sidx = within % S;
  const int b = gi / HG, hg = gi - b * HG;
  // query row b reads cache bc (its rows, length and window); its query,
  // index list, position, partials and output are its own
  const int bc = qps == 1 ? b : b / qps;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int kw = WF8 ? (k + 15) & ~15 : k;  // first window slot
  const int nslots = kw + swa_cap;

  // ---- loads: index entry, lengths and the 16 queries (to LDS, 32 B per
  // thread), then the row.  Every load is unconditional (clamped addresses,
  // results masked afterwards): a conditional load makes the compiler wait
  // for it where the branches join.  The lengths are per-lane vector loads
  // (a scalar load is waited for before the next one is issued); a NULL
  // pointer reads the query instead and counts as 0.
  int vzero;  // an opaque 0 in a VGPR: keeps the length loads on the vector path
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  const int slot = kRows * sidx + 16 * w + n;
  // the wave's 16 slots are all selected entries or all window records
  // (kw is a multiple of 16): its query fragments follow that row layout,
  // whether or not each of its rows is visible
  const bool wwin = WF8 && kRows * sidx + 16 * w >= kw;
  const int32_t* tp = k > 0 ? topk + (int64_t)b * k + min(slot, k - 1) : reinterpret_cast<const int32_t*>(q);
  const int32_t praw = tp[0];
  const int32_t Lraw = (len ? len + bc : reinterpret_cast<const int32_t*>(q))[vzero];
  const int32_t SLraw = (swa_len ? swa_len + bc : reinterpret_cast<const int32_t*>(q))[vzero];
  const uint4* qg = reinterpret_cast<const uint4*>(q + ((int64_t)b * H + 16 * hg) * 512);
  // 16 heads x 64 pieces of 16 B: two pieces per thread
  static_assert(kThreads >= 512 && kThreads < 1024, "two query pieces per thread");
  uint4 qv0 = qg[tid];
  uint4 qv1 = qg[min(tid + kThreads, 1023)];
  const int64_t qpos = (q_pos ? q_pos + b : reinterpret_cast<const int64_t*>(q))[vzero];
  // Touch the 128 lines of this chunk's partial (16 heads x 1 KB): gfx950's
  // L2 does not allocate a line on a write miss, so without this the partial
  // stores go to memory and the merge reads them back from there; with the
  // lines resident the stores update them and the merge finds them in L2.
  // The loads complete during the row loads and are consumed, unused, by the
  // partial stores.
  uint32_t touch = 0u;
  if (tid < 128)
    touch = reinterpret_cast<const uint32_t*>(
        part + (((int64_t)b * H + 16 * hg + (tid >> 3)) * S + sidx) * 512 + 64 * (tid & 7))[0];
  // all of the above in flight together: the compiler would otherwise sink
  // each load into the branch that uses it and wait for them one by one
  asm volatile("" ::"v"(praw), "v"(Lraw), "v"(SLraw), "v"(qpos));
  const int32_t pidx = slot < k ? praw : -1;
  if (!valid) return;
  if constexpr (F16) {
    // decoded E4M3 scale bytes, one table entry per byte value (built while
    // the loads above are in flight; read after the query barrier)
    if (tid < 256) {
      const E4m3F16 e = e4m3_f16_scale((uint32_t)tid);
      sm.e4lut[tid] = make_uint2(__float_as_uint(e.pow2), __builtin_bit_cast(uint32_t, e.sig));
    }
  }
  int64_t L = len ? Lraw : cap;  // no lengths: absolute row ids below cap
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int SL = swa_len ? SLraw : 0;
  SL = SL < 0 ? 0 : (SL > swa_cap ? swa_cap : SL);
  RowFetch row;
  {
    const RowSrc src = locate_row<WF8>(slot, pidx, nslots, bc, k, kw, L, SL, seq_stride, swa_stride, main_codes,
                                       main_scales, swa_codes, swa_scales);
    if constexpr (WF8)
      fetch_row_w8(row, src, g);
    else
      fetch_row(row, src, g);
  }
  // with 8 waves the query tile borrows the R buffer, which is then not
  // written before the max barrier
  uint16_t* Q = Smem::kQOwn ? sm.Qown : sm.R;
  if (q_pos) {  // Q RoPE: pieces 56..63 of a head hold dims 448..511
    if ((tid & 63) >= 56) qv0 = rope_bf16x8(qv0, 8 * (tid & 63), qpos);
    if (((tid + kThreads) & 63) >= 56) qv1 = rope_bf16x8(qv1, 8 * ((tid + kThreads) & 63), qpos);
  }
  if constexpr (F16) {
    // fp16 query: each wave holds whole heads (qv0: head tid/64; qv1: head
    // (tid + kThreads)/64, for whole waves), scaled by 2^-k into fp16 range;
    // the logits take 2^k back
    const int k0 = head_shift_f16(qv0);
    qv0 = bf16x8_to_f16_scaled(qv0, k0);
    if (lane == 0) sm.qk[tid >> 6] = k0;
    if (tid + kThreads < 1024) {  // wave-uniform
      const int k1 = head_shift_f16(qv1);
      qv1 = bf16x8_to_f16_scaled(qv1, k1);
      if (lane == 0) sm.qk[(tid + kThreads) >> 6] = k1;
    }
  }
  *reinterpret_cast<uint4*>(&Q[(tid >> 6) * kQLd + 8 * (tid & 63)]) = qv0;
  if (tid + kThreads < 1024) {
    const int e = tid + kThreads;
    *reinterpret_cast<uint4*>(&Q[(e >> 6) * kQLd + 8 * (e & 63)]) = qv1;
  }
  __syncthreads();

  // ---- logits of the wave's 16 rows (every row dequantised once, kept for P.R)
  // staged row of this lane and the units of its K steps in each half-row:
  // K step ks (< 8) is dims 64g+8ks (unit 8g+ks); K step 8+ks is dims
  // 256+64g+8ks, or for an FP8 window record 256+48g+8ks (ks < 6) and
  // 448+16g+8(ks-6) (units 6g+ks and 24+2g+ks-6 of the second half-row)
  const int rr = 16 * w + n;
  auto h0unit = [&](int ks) -> int { return 8 * g + ks; };
  auto h1unit = [&](int ks) -> int {
    if (wwin) return ks < 6 ? 6 * g + ks : 24 + 2 * g + (ks - 6);
    return 8 * g + ks;
  };
  floatx4 sacc = floatx4{0.f, 0.f, 0.f, 0.f};
  V8 ra[16];
  // query fragments of kQB K steps are read before their products (fewer at
  // 8 waves, where four waves share a SIMD and registers are scarcer)
  constexpr int kQB = Smem::kQOwn ? 8 : 4;
#pragma unroll
  for (int kb = 0; kb < 16; kb += kQB) {
    V8 qf[kQB];
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const int dq = wwin ? step_dim_w8(kb + j, g) : step_dim(kb + j, g);
      qf[j] = *reinterpret_cast<const V8*>(&Q[n * kQLd + dq]);
    }
    uint2 lt[kQB / 2];  // fp16 path: decoded scales of the batch's pairs of K steps
    if constexpr (F16) {
#pragma unroll
      for (int j = 0; j < kQB / 2; ++j) lt[j] = sm.e4lut[row_scale_byte(row, kb + 2 * j)];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      if constexpr (F16) {
        const E4m3F16 sc16{__uint_as_float(lt[j >> 1].x), __builtin_bit_cast(f16x2, lt[j >> 1].y)};
        ra[kb + j] = row_step_f16(row, kb + j, sc16);
      } else if constexpr (WF8)
        ra[kb + j] = wwin ? row_step_w8(row, kb + j, g) : row_step<FMT>(row, kb + j);
      else
        ra[kb + j] = row_step<FMT>(row, kb + j);
      sacc = mfma16<F16>(ra[kb + j], qf[j], sacc);
    }
  }
  if (Smem::kQOwn) {
    // the first half of the wave's rows goes to LDS now (R is not shared with Q)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) *reinterpret_cast<V8*>(&sm.R[runit(rr, h0unit(ks))]) = ra[ks];
  }
  // lane (g, n): rows 4g+i of the wave's tile, head n; fp16 queries were
  // staged times 2^-qk[n]
  const uint64_t vmask = __ballot(row.ok != 0u);
  // (fp16: scaled back by 2^k after sm_scale, so the logit overflows only
  // when its true value does)
  const int qk = F16 ? sm.qk[n] : 0;
  float x[4];
  float mw = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float xs = F16 ? ldexpf(sacc[i] * sm_scale, qk) : sacc[i] * sm_scale;
    x[i] = ((vmask >> (4 * g + i)) & 1ull) ? xs : -INFINITY;
    mw = fmaxf(mw, x[i]);
  }
  mw = rows4_max(mw);
  if (g == 0) sm.red_m[w][n] = mw;
  {
    // largest scale byte of the lane's 128 values -> bound of |value| (6 x scale)
    uint32_t mb = 0u;
#pragma unroll
    for (int q4 = 0; q4 < 8; ++q4) {
      const uint32_t by = (row.s[q4 >> 2] >> (8 * (q4 & 3))) & 0xFFu;
      mb = max(mb, (FMT == 0 || (WF8 && row.win)) ? by : (by & 0x7Fu));  // positive E4M3 bytes order like values
    }
    float vb = row.ok ? 6.0f * (FMT == 0 ? e8m0_value(mb) : e4m3_value(mb)) : 0.0f;
    if (WF8 && row.win) {
      // E4M3 dims: 448 x the largest scale; bf16 dims: their own magnitudes
      float rm = 0.0f;
#pragma unroll
      for (int j = 3; j < 5; ++j) {
        const uint32_t wd[4] = {row.x[j].x, row.x[j].y, row.x[j].z, row.x[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          rm = fmaxf(rm, fmaxf(fabsf(bf16_bits_to_f32(wd[i] & 0xFFFFu)), fabsf(bf16_bits_to_f32(wd[i] >> 16))));
      }
      vb = fmaxf(448.0f * e8m0_value(mb), rm);
    }
    if (!(vb <= 3.0e38f)) vb = 3.0e38f;  // NaN/inf scale bytes: clamp the bound
    vb = wave_max(vb);
    if (lane == 0) sm.red_v[w] = vb;
  }
  __syncthreads();  // also: every wave is done reading the query tile
  float M = sm.red_m[0][n];
#pragma unroll
  for (int v = 1; v < WAVES; ++v) M = fmaxf(M, sm.red_m[v][n]);
  float lw = 0.f;
  float pf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pf[i] = (M == -INFINITY) ? 0.0f : __expf(x[i] - M);
    lw += pf[i];
  }
  lw = rows4_sum(lw);
  if (g == 0) sm.red_l[w][n] = lw;
  // slots 16w + 4g .. +3: unit 2w + g/2, plane g & 1
  *reinterpret_cast<uint2*>(&sm.P[(g & 1) * 16 * kPP + n * kPP + 4 * (2 * w + (g >> 1))]) =
      F16 ? make_uint2(pack_f16x2(pf[0], pf[1]), pack_f16x2(pf[2], pf[3]))
          : make_uint2(pack_bf16x2(pf[0], pf[1]), pack_bf16x2(pf[2], pf[3]));
  if (!Smem::kQOwn) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) *reinterpret_cast<V8*>(&sm.R[runit(rr, h0unit(ks))]) = ra[ks];
  }
  __syncthreads();

  uint16_t* prow = part + ((int64_t)b * H + 16 * hg) * S * 512;
  asm volatile("" ::"v"(touch));
  const uint32_t my_xcc = __builtin_amdgcn_s_getreg(kHwRegXccId);
  // The partial is stored as fp16 of (output / sum) * 2^-e: a convex
  // combination of the chunk's rows, so |.| <= vmax, and 2^e brings vmax
  // just under 2^15 (fp16 keeps 11 significant bits).
  float vmax = sm.red_v[0];
#pragma unroll
  for (int v = 1; v < WAVES; ++v) vmax = fmaxf(vmax, sm.red_v[v]);
  int e_sc = 0;  // vmax < 2^(e_sc + 15)
  if (vmax > 0.0f) {
    int ex;
    (void)frexpf(vmax, &ex);
    e_sc = ex - 15;
  }
  if (w == 0 && g == 0) {
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) l += sm.red_l[v][n];
    ml[((int64_t)b * H + 16 * hg + n) * S + sidx] =
        make_float4(M, l, __uint_as_float(my_xcc), __int_as_float(e_sc));
  }
  // 1 / sum for heads 4g+i (a reciprocal: the sum is >= 1 when positive);
  // the partial's 2^-e is applied per value (2^-e alone can exceed fp32)
  float scl;  // 1 / sum for head n
  {
    float ln = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) ln += sm.red_l[v][n];
    scl = ln > 0.f ? __builtin_amdgcn_rcpf(ln) : 0.0f;
  }
  V8 pa[kRows / 32];  // P operands, read once for both halves (one workgroup per CU)
  if constexpr (Smem::kQOwn) {
#pragma unroll
    for (int kk = 0; kk < kRows / 32; ++kk) pa[kk] = p_operand<WAVES, F16>(sm, kk, g, n);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 1) {
      __syncthreads();  // every wave is done reading the first half
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) *reinterpret_cast<V8*>(&sm.R[runit(rr, h1unit(ks))]) = ra[8 + ks];
      __syncthreads();
    }
    floatx4 O[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    pv_half<WAVES, F16>(sm, w, g, n, pa, O);
    // lane (g, n): head n, dims 256h + 16*tile + 4g .. +3, tile = w + WAVES*nt:
    // one 8-byte store per tile
    uint2* dst = reinterpret_cast<uint2*>(prow + ((int64_t)n * S + sidx) * 512 + 256 * h + 16 * w + 4 * g);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (nt == 1 && w + WAVES >= 16) break;  // wave-uniform
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ldexpf(O[nt][i] * scl, -e_sc);
      dst[nt * 4 * WAVES] = make_uint2(pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]));
    }
  }

  // ---- the last chunk of the group to finish merges all S partials
  if (!arrive_last(cnt + gi, (uint32_t)S, &sm.last)) return;  // workgroup-uniform
  if (tid < 16 * 32) {
    if (q_pos)
      merge_splits<true>(b, 16 * hg, H, S, ml, part, out, lse, my_xcc, tid, merge_rope(q_pos[b], tid & 31));
    else
      merge_splits<false>(b, 16 * hg, H, S, ml, part, out, lse, my_xcc, tid, MergeRope{});
  }
}


// ===================================================== throughput variant
// One workgroup per (sequence, split of 32-row chunks) takes all 64 heads,
// so every row is dequantised and staged once (the split kernel above does it
// once per 16-head group), and it loops over its chunks with an online
// softmax instead of ending after one chunk.  Used where the batch alone
// fills the chip; the split kernel keeps the decode latency at small batch.
//  * Eight waves in two roles, one of each per SIMD.  Score waves (0..3):
//    wave w owns heads 16w..16w+15, keeps their queries in registers as MFMA
//    B operands (K step ks: dims 32ks + 8g..+7 in lane group g), computes
//    S = R.Q^T from the staged rows and the online softmax, and writes P
//    (bf16) and the per-head rescale factor to LDS.  Value waves (4..7):
//    wave 4+v owns dims 128v..128v+127 of every head, computes
//    O^T += R^T.P^T one chunk behind the score waves, and stages the rows.
//    The two roles overlap on each SIMD; one barrier per chunk.
//  * Rows live in a ring of three 32-row buffers (chunk c+1 being staged,
//    c being scored, c-1 being multiplied).  A step takes about 1 us while a
//    loaded row arrives 2-3 us after its index entry is known under full
//    load, so rows are loaded three chunks ahead of staging.  Index entries
//    are loaded seven chunks ahead: loads complete in order, so waiting for
//    an index entry also waits for every row load issued before it, and
//    those must be old by then.
//  * Staged rows are 1 KB apart; 16-byte unit u of row r is stored at unit
//    u ^ swz(r mod 16), swz(x) = x ^ ((x >> 2) << 1), which keeps the row
//    reads of Q.R^T free of bank conflicts (measured on gfx950).
//  * S = R.Q^T leaves lane (g, n) with rows 4g..4g+3 of each 16-row tile for
//    head n; P is stored per head in the K-slot order of the 32-row P.R
//    MFMA (lane group g: rows 4g + 0..3, then 16 + 4g + 0..3), so each B
//    operand is one 16-byte read.  R^T comes from ds_read_b64_tr_b16 in the
//    same row order.
//  * The running maximum moves only when a chunk exceeds it by more than
//    2^8 (P <= 256 in between), so the accumulators are rarely rescaled.
//  * FP8 window records (576 data + 8 scale bytes) are staged 16 rows per
//    chunk, so that 16 staging lanes of 36 bytes cover a record and every
//    lane keeps its load slot; the lane's scale byte arrives through the
//    index-entry slot, which a window chunk does not otherwise use.
constexpr int kTRows = 32;     // rows per chunk
constexpr int kTRowB = 1024;   // staged row: 512 bf16
constexpr int kTPLd = 40;      // P row stride in bf16 (32 slots + pad)
constexpr float kTau = 8.0f;   // log2 headroom before the running max moves

__device__ __forceinline__ int tswz(int r) {
  r &= 15;
  return r ^ ((r >> 2) << 1);
}

struct AttnTSmem {
  uint8_t R[3][kTRows * kTRowB];
  uint16_t P[2][64 * kTPLd];
  float alpha[2][64];  // rescale factor per head for the chunk in P[.]
  float mfin[64], lfin[64];
  uint32_t vb[3];      // row validity of the chunk in R[.]
  float red_v[4];
  int last;
};

// The staging lane's slice of one row: 32 code bytes and 4 scale bytes.
struct TStage {
  uint4 c0, c1;
  uint32_t s;
  uint32_t ok;
};

template <int FMT, bool WF8>
__global__ __launch_bounds__(512, 1) void attn_seq_kernel(
    const uint16_t* __restrict__ q, int H, const uint8_t* __restrict__ main_codes,
    const uint8_t* __restrict__ main_scales, int64_t cap, const int32_t* __restrict__ len,
    const int32_t* __restrict__ topk, int k, const uint8_t* __restrict__ swa_codes,
    const uint8_t* __restrict__ swa_scales, int64_t swa_stride, int swa_cap,
    const int32_t* __restrict__ swa_len, float sm_scale, const int64_t* __restrict__ q_pos, int B, int S,
    uint16_t* __restrict__ part, float4* __restrict__ ml, uint32_t* __restrict__ cnt,
    uint16_t* __restrict__ out, float* __restrict__ lse, int64_t seq_stride, int qps) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnTSmem& sm = *reinterpret_cast<AttnTSmem*>(smem_raw);
  asm volatile("" ::"s"(q), "s"(main_codes), "s"(main_scales), "s"(len), "s"(topk), "s"(swa_codes),
               "s"(swa_scales), "s"(swa_len), "s"(part), "s"(ml), "s"(cnt), "s"(out), "s"(lse),
               "s"(H), "s"(cap), "s"(k), "s"(swa_stride), "s"(swa_cap), "s"(sm_scale), "s"(B), "s"(S), "s"(qps));
  // the S workgroups of a sequence get ids congruent mod 8 (one XCD), so the
  // partials the last one merges are in its L2
  const int id = blockIdx.x, xcd = id & 7, r8 = id >> 3;
  const int b = (r8 / S) * 8 + xcd, sidx = r8 % S;
  if (b >= B) return;  // padding workgroup (uniform, before any barrier)
  // query row b reads cache bc (its rows, length and window); its query,
  // index list, position, partials and output are its own
  const int bc = qps == 1 ? b : b / qps;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const bool scorer = w < 4;  // wave-uniform role
  const int wr = w & 3;       // index within the role
  const int nslots = k + swa_cap;
  // FP8 window records: the selected entries fill 32-row chunks up to kw (k
  // rounded up to 32), then the window takes 16-row chunks -- a record is
  // twice a main entry, so 16 lanes of 36 bytes stage one row and every
  // staging lane keeps the same load slot
  const int kw = WF8 ? (k + 31) & ~31 : k;
  const int kwc = kw / kTRows;  // first window chunk (FP8 records)
  const int nch = WF8 ? kwc + (swa_cap + 15) / 16 : (nslots + kTRows - 1) / kTRows;
  const int c_begin = (int)((int64_t)sidx * nch / S), c_end = (int)((int64_t)(sidx + 1) * nch / S);
  const int nc = c_end - c_begin;
  // steps of the chunk loop, rounded up to the value waves' unroll of three
  // (the extra steps only synchronise); both roles run exactly this many
  const int nsteps = (nc + 1 + 2) / 3 * 3;

  int64_t L = len ? len[bc] : cap;  // no lengths: absolute row ids below cap
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int SL = swa_len ? swa_len[bc] : 0;
  SL = SL < 0 ? 0 : (SL > swa_cap ? swa_cap : SL);

  // ---- value waves: staging role, row srow of a chunk, dims 64*ssp .. +63;
  // in an FP8 window chunk, row wrow, bytes 32*wt .. +31 and 512 + 4*wt .. +3
  const int srow = 16 * (wr & 1) + n, ssp = 4 * (wr >> 1) + g;
  const int wrow = (64 * wr + lane) >> 4, wt = lane & 15;
  const int32_t* tbase = topk + (int64_t)b * k;
  const uint8_t* dummy = reinterpret_cast<const uint8_t*>(q + (int64_t)b * H * 512);
  // raw index-list entry of row srow of chunk c, loaded unconditionally from
  // a clamped address (a valid dummy when k = 0).  It is not tested here:
  // anything computed from it right away would make the compiler wait for
  // the load at once.  load_rows applies every validity condition.
  // In an FP8 window chunk the slot carries the scale dword holding the
  // lane's group byte instead (group wt/2 of row wrow), from the same clamped
  // kind of address.
  auto load_idx = [&](int c) -> int32_t {
    const int slot = c * kTRows + srow;
    const int32_t* ip = k > 0 ? tbase + min(slot, k - 1) : reinterpret_cast<const int32_t*>(dummy);
    if (WF8 && c >= kwc) {
      const int rr = (c - kwc) * 16 + wrow;
      ip = rr < SL ? reinterpret_cast<const int32_t*>(swa_scales + ((int64_t)bc * swa_stride + rr) * kWinScaleB +
                                                      4 * ((wt >> 1) >> 2))
                   : reinterpret_cast<const int32_t*>(dummy);
    }
    return *ip;
  };
  auto load_rows = [&](int c, int32_t p) -> TStage {
    const int slot = c * kTRows + srow;
    const uint8_t* cp = dummy;
    const uint8_t* scp = dummy;
    uint32_t ok = 0u;
    if (c < c_end) {
      if (slot < k) {
        if (p >= 0 && (int64_t)p < L) {
          cp = main_codes + ((int64_t)bc * seq_stride + p) * 256;
          scp = main_scales + ((int64_t)bc * seq_stride + p) * 32;
          ok = 1u;
        }
      } else if (!WF8 && slot < nslots && slot - k < SL) {
        cp = swa_codes + ((int64_t)bc * swa_stride + (slot - k)) * 256;
        scp = swa_scales + ((int64_t)bc * swa_stride + (slot - k)) * 32;
        ok = 1u;
      }
    }
    const uint8_t* a0 = cp + 32 * ssp;
    const uint8_t* as = scp + 4 * ssp;
    if (WF8 && c >= kwc) {
      // FP8 window record: bit 0 of ok = visible, bits 8..15 = the scale byte
      const int rr = (c - kwc) * 16 + wrow;
      const bool vis = c < c_end && rr < SL;
      cp = vis ? swa_codes + ((int64_t)bc * swa_stride + rr) * kWinDataB : dummy;
      a0 = cp + 32 * wt;
      as = cp + 512 + 4 * wt;
      ok = vis ? 1u | ((((uint32_t)p >> (8 * ((wt >> 1) & 3))) & 0xFFu) << 8) : 0u;
    }
    TStage st;
    const uint4* c4 = reinterpret_cast<const uint4*>(a0);
    st.c0 = c4[0];
    st.c1 = c4[1];
    st.s = *reinterpret_cast<const uint32_t*>(as);
    st.ok = ok;
    return st;
  };
  uint32_t smax = 0u;  // largest scale byte staged by this lane (bound of |value|)
  float wmax = 0.0f;   // bound of |value| of the FP8 window records it staged
  const int wsw = tswz(srow);
  // FP8 window chunk j: rows 0..15 of R[buf] from the records (invisible ones
  // as zeros), rows 16..31 zero; validity from the window length
  auto stage_win = [&](int buf, TStage st, int j) {
    const uint32_t m = 0u - (st.ok & 1u);
    st.c0 = make_uint4(st.c0.x & m, st.c0.y & m, st.c0.z & m, st.c0.w & m);
    st.c1 = make_uint4(st.c1.x & m, st.c1.y & m, st.c1.z & m, st.c1.w & m);
    st.s &= m;
    uint8_t* rowp = sm.R[buf] + wrow * kTRowB;
    const int sw = tswz(wrow);
    auto bmax = [](uint32_t v) {
      return fmaxf(fabsf(bf16_bits_to_f32(v & 0xFFFFu)), fabsf(bf16_bits_to_f32(v >> 16)));
    };
    if (wt < 14) {
      const uint32_t sb = (st.ok >> 8) & 0xFFu;
      const float op = e8m0_operand(sb);
      const uint32_t cw[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *reinterpret_cast<bf16x8*>(rowp + (((4 * wt + u) ^ sw) << 4)) = fp8x8_to_bf16(cw[2 * u], cw[2 * u + 1], op);
      if (st.ok & 1u) wmax = fmaxf(wmax, 448.0f * e8m0_value(sb));
    } else {
      *reinterpret_cast<uint4*>(rowp + (((56 + 2 * (wt - 14)) ^ sw) << 4)) = st.c0;
      *reinterpret_cast<uint4*>(rowp + (((57 + 2 * (wt - 14)) ^ sw) << 4)) = st.c1;
      wmax = fmaxf(wmax, fmaxf(fmaxf(fmaxf(bmax(st.c0.x), bmax(st.c0.y)), fmaxf(bmax(st.c0.z), bmax(st.c0.w))),
                               fmaxf(fmaxf(bmax(st.c1.x), bmax(st.c1.y)), fmaxf(bmax(st.c1.z), bmax(st.c1.w)))));
    }
    // dims 480 + 2wt, 481 + 2wt: a quarter of unit 60 + wt/4
    *reinterpret_cast<uint32_t*>(rowp + (((60 + (wt >> 2)) ^ sw) << 4) + 4 * (wt & 3)) = st.s;
    wmax = fmaxf(wmax, bmax(st.s));
    uint8_t* zrow = sm.R[buf] + (16 + wrow) * kTRowB;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(zrow + ((4 * wt + u) << 4)) = make_uint4(0u, 0u, 0u, 0u);
    if (wr == 0 && lane == 0) {
      const int nv = min(max(SL - 16 * j, 0), 16);
      sm.vb[buf] = nv >= 16 ? 0xFFFFu : ((1u << nv) - 1u);
    }
  };
  // dequantise the lane's slice into R[buf] (invalid rows as zeros) and
  // record the chunk's row validity
  auto stage = [&](int buf, TStage st, int c) {
    if (WF8 && c >= kwc) {
      stage_win(buf, st, c - kwc);
      return;
    }
    const uint32_t m = 0u - st.ok;
    st.c0 = make_uint4(st.c0.x & m, st.c0.y & m, st.c0.z & m, st.c0.w & m);
    st.c1 = make_uint4(st.c1.x & m, st.c1.y & m, st.c1.z & m, st.c1.w & m);
    st.s &= m;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t by = (st.s >> (8 * j)) & 0xFFu;
      smax = max(smax, FMT == 0 ? by : (by & 0x7Fu));  // positive E4M3 bytes order like values
    }
    const uint32_t cw[8] = {st.c0.x, st.c0.y, st.c0.z, st.c0.w, st.c1.x, st.c1.y, st.c1.z, st.c1.w};
    uint8_t* rowp = sm.R[buf] + srow * kTRowB;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<bf16x8*>(rowp + (((8 * ssp + j) ^ wsw) << 4)) =
          dequant8<FMT>(cw[j], (st.s >> (8 * (j >> 1))) & 0xFFu);
    const uint64_t bal = __ballot(st.ok != 0u);
    if (wr < 2 && lane == 0) reinterpret_cast<uint16_t*>(&sm.vb[buf])[wr] = (uint16_t)(bal & 0xFFFFull);
  };

  // The two roles run separate loops with the same number of barriers (one
  // per step, plus the prologue's and the final one), so each keeps only its
  // own state live: the queries in the score waves, the output in the value
  // waves.
  const uint32_t my_xcc = __builtin_amdgcn_s_getreg(kHwRegXccId);
  if (scorer) {
    // ---- queries of heads 16wr .. +15 (lane (g, n): head 16wr + n)
    bf16x8 qf[16];
    {
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)b * H + 16 * wr + n) * 512 + 8 * g);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, qp[4 * ks]);
      if (q_pos) {  // Q RoPE: K steps 14 and 15 hold dims 448..511
        const int64_t pos = q_pos[b];
#pragma unroll
        for (int ks = 14; ks < 16; ++ks)
          qf[ks] = __builtin_bit_cast(bf16x8, rope_bf16x8(__builtin_bit_cast(uint4, qf[ks]), 32 * ks + 8 * g, pos));
      }
    }
    float mref = -INFINITY, lsum = 0.f;  // softmax of head 16wr + n (lane partial sum)
    const float c2 = sm_scale * 1.4426950408889634f;  // logits in log2 units
    // row 16t + n, unit 4ks + g -> qoff[ks%4] + 256*(ks/4) + 16384t
    int qoff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qoff[m] = n * kTRowB + (((4 * m + g) ^ tswz(n)) << 4);
    __syncthreads();  // chunk c_begin staged
    for (int s = 0; s < nsteps; ++s) {  // step s: score chunk s
      if (s < nc) {
        const uint8_t* Rb = sm.R[s % 3];
        const uint32_t vm = sm.vb[s % 3];
        // ---- S = R . Q^T for the chunk's two 16-row tiles; reads two K steps ahead
        floatx4 sacc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
        bf16x8 qa[3][2];
        auto qk_read = [&](int slot, int ks) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            qa[slot][t] = *reinterpret_cast<const bf16x8*>(Rb + qoff[ks & 3] + 256 * (ks >> 2) + 16384 * t);
        };
        qk_read(0, 0);
        qk_read(1, 1);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          if (ks + 2 < 16) qk_read((ks + 2) % 3, ks + 2);
#pragma unroll
          for (int t = 0; t < 2; ++t) sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks % 3][t], qf[ks], sacc[t], 0, 0, 0);
        }
        // ---- online softmax (lane (g, n): rows 16t + 4g + i, head 16wr + n)
        float x[8];
        float cmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * t + 4 * g + i;
            x[4 * t + i] = ((vm >> row) & 1u) ? sacc[t][i] * c2 : -INFINITY;
            cmax = fmaxf(cmax, x[4 * t + i]);
          }
        cmax = rows4_max(cmax);
        float alpha = 1.0f;
        if (cmax > mref + kTau) {
          alpha = mref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mref - cmax);
          mref = cmax;
          lsum *= alpha;
        }
        const float mu = mref == -INFINITY ? 0.0f : mref;
        float pf[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // x = -inf (masked row) gives 0; x - mu <= kTau
          pf[j] = __builtin_amdgcn_exp2f(x[j] - mu);
          lsum += pf[j];
        }
        // slots 8g + 4t + i = rows 16t + 4g + i
        *reinterpret_cast<uint4*>(sm.P[s & 1] + (16 * wr + n) * kTPLd + 8 * g) =
            make_uint4(pack_bf16x2(pf[0], pf[1]), pack_bf16x2(pf[2], pf[3]), pack_bf16x2(pf[4], pf[5]),
                       pack_bf16x2(pf[6], pf[7]));
        if (g == 0) sm.alpha[s & 1][16 * wr + n] = alpha;
      }
      __syncthreads();
    }
    lsum = rows4_sum(lsum);
    if (g == 0) {
      sm.mfin[16 * wr + n] = mref;
      sm.lfin[16 * wr + n] = lsum;
    }
    __syncthreads();  // final softmax state of every head in LDS
  } else {
    // ---- prologue: stage chunk c_begin; rows of c_begin+1 .. +3 and index
    // entries of c_begin+4 .. +6 in flight.  Slot j of XA/XB/XC and PA/PB/PC
    // serves the steps s = j mod 3 (rows of chunk s+1, index entries of
    // chunk s+4); the step loop is unrolled by three so that no register
    // holding an outstanding load is ever copied (a copy would wait for it).
    TStage XA, XB, XC;
    int32_t PA, PB, PC;
    {
      // issue order as in the steady state (rows of chunk j, then the index
      // entry of chunk j+3), so that the loop's waits count the same loads
      const int32_t p0 = load_idx(c_begin);
      const int32_t p1 = load_idx(c_begin + 1);
      const int32_t p2 = load_idx(c_begin + 2);
      const int32_t p3 = load_idx(c_begin + 3);
      const TStage st0 = load_rows(c_begin, p0);
      XA = load_rows(c_begin + 1, p1);
      PA = load_idx(c_begin + 4);
      XB = load_rows(c_begin + 2, p2);
      PB = load_idx(c_begin + 5);
      XC = load_rows(c_begin + 3, p3);
      PC = load_idx(c_begin + 6);
      stage(0, st0, c_begin);
    }
    // O^T tile (dims 128wr + 16dt .., heads 16ht ..): lane (g, n) holds dims
    // +4g..+3 of head 16ht + n
    floatx4 O[8][4];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) O[dt][ht] = floatx4{0.f, 0.f, 0.f, 0.f};
    // A = R^T: row 4g + n/4 (+16), dims 128wr + 16dt + 4(n&3)
    int toff[8];
    {
      const int tr = 4 * g + (n >> 2), ta = n & 3;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        toff[dt] = tr * kTRowB + 256 * wr + (((2 * dt + (ta >> 1)) ^ tswz(tr)) << 4) + 8 * (ta & 1);
    }
    __syncthreads();  // chunk c_begin staged
    // step s: stage chunk s+1 (rows in X), multiply chunk s-1, then load the
    // rows of chunk s+4 (index entry in Pn) and the index entries of chunk s+7.
    // Staging first puts the value wave's conversions beside the score wave's
    // products on the same SIMD (R[(s+1)%3] was last read in step s-1).
    auto vstep = [&](int s, TStage& X, int32_t& Pn) {
      if (s + 1 < nc) stage((s + 1) % 3, X, c_begin + s + 1);
      if (s >= 1 && s <= nc) {
        // ---- O^T(dims of this wave, all heads) += R^T . P^T for chunk s-1
        const uint8_t* Rb = sm.R[(s - 1) % 3];
        const uint16_t* Pb = sm.P[(s - 1) & 1];
        float al[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) al[ht] = sm.alpha[(s - 1) & 1][16 * ht + n];
        if (__ballot(al[0] != 1.0f || al[1] != 1.0f || al[2] != 1.0f || al[3] != 1.0f) != 0ull) {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) O[dt][ht] *= al[ht];
        }
        bf16x8 pbv[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) pbv[ht] = *reinterpret_cast<const bf16x8*>(Pb + (16 * ht + n) * kTPLd + 8 * g);
        shortx4 tq[3][2];
        auto tr_read = [&](int slot, int dt) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            tq[slot][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) shortx4*)(Rb + toff[dt] + kTRowB * 16 * hh));
        };
        tr_read(0, 0);
        tr_read(1, 1);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          if (dt + 2 < 8) tr_read((dt + 2) % 3, dt + 2);
          const shortx4 lo = tq[dt % 3][0], hi = tq[dt % 3][1];
          shortx8 av;
          av[0] = lo[0]; av[1] = lo[1]; av[2] = lo[2]; av[3] = lo[3];
          av[4] = hi[0]; av[5] = hi[1]; av[6] = hi[2]; av[7] = hi[3];
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
            O[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pbv[ht], O[dt][ht], 0, 0, 0);
        }
      }
      // issued on every step (past the split they read a dummy row), so that
      // the count of outstanding loads is the same on every path and each
      // wait covers only the loads it needs
      X = load_rows(c_begin + s + 4, Pn);
      Pn = load_idx(c_begin + s + 7);
      __syncthreads();
    };
    for (int s0 = 0; s0 < nsteps; s0 += 3) {
      vstep(s0, XA, PA);
      vstep(s0 + 1, XB, PB);
      vstep(s0 + 2, XC, PC);
    }
    if (S > 1) {
      float vb = 6.0f * (FMT == 0 ? e8m0_value(smax) : e4m3_value(smax));
      if (WF8) vb = fmaxf(vb, wmax);
      if (!(vb <= 3.0e38f)) vb = 3.0e38f;  // NaN/inf scale bytes: clamp the bound
      vb = wave_max(vb);
      if (lane == 0) sm.red_v[wr] = vb;
    }
    __syncthreads();  // final softmax state of every head in LDS
    float hm[4], hl[4], inv[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
      hm[ht] = sm.mfin[16 * ht + n];
      hl[ht] = sm.lfin[16 * ht + n];
      inv[ht] = hl[ht] > 0.f ? __builtin_amdgcn_rcpf(hl[ht]) : 0.0f;  // the sum is >= 1 when positive
    }
    if (S == 1) {
      if (q_pos && wr == 3) {
        // output inverse RoPE: dims 448 + 16(dt-4) + 4g + 0..3 are pairs 8(dt-4) + 2g + 0..1
        const int64_t pos = q_pos[b];
#pragma unroll
        for (int dt = 4; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            float c, sn;
            rope_cos_sin(pos, 8 * (dt - 4) + 2 * g + i, c, sn);
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
              float x0 = O[dt][ht][2 * i], x1 = O[dt][ht][2 * i + 1];
              rope_pair<true>(x0, x1, c, sn);
              O[dt][ht][2 * i] = x0;
              O[dt][ht][2 * i + 1] = x1;
            }
          }
      }
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        uint16_t* orow = out + ((int64_t)b * H + 16 * ht + n) * 512 + 128 * wr + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<uint2*>(orow + 16 * dt) =
              make_uint2(pack_bf16x2(O[dt][ht][0] * inv[ht], O[dt][ht][1] * inv[ht]),
                         pack_bf16x2(O[dt][ht][2] * inv[ht], O[dt][ht][3] * inv[ht]));
        if (lse && wr == 0 && g == 0)
          lse[(int64_t)b * H + 16 * ht + n] =
              hl[ht] > 0.f ? (hm[ht] + log2f(hl[ht])) * 0.6931471805599453f : -INFINITY;
      }
    } else {
      // partial: fp16 of (output / sum) * 2^-e, |output / sum| <= vmax < 2^(e + 15)
      const float vmax = fmaxf(fmaxf(sm.red_v[0], sm.red_v[1]), fmaxf(sm.red_v[2], sm.red_v[3]));
      int e_sc = 0;
      if (vmax > 0.0f) {
        int ex;
        (void)frexpf(vmax, &ex);
        e_sc = ex - 15;
      }
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const int64_t bh = (int64_t)b * H + 16 * ht + n;
        uint16_t* prow = part + (bh * S + sidx) * 512 + 128 * wr + 4 * g;
        const float sc = inv[ht];  // the partial's 2^-e is applied per value (2^-e alone can exceed fp32)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<uint2*>(prow + 16 * dt) =
              make_uint2(pack_f16x2(ldexpf(O[dt][ht][0] * sc, -e_sc), ldexpf(O[dt][ht][1] * sc, -e_sc)),
                         pack_f16x2(ldexpf(O[dt][ht][2] * sc, -e_sc), ldexpf(O[dt][ht][3] * sc, -e_sc)));
        if (wr == 0 && g == 0)
          ml[bh * S + sidx] = make_float4(hm[ht] == -INFINITY ? -INFINITY : hm[ht] * 0.6931471805599453f, hl[ht],
                                          __uint_as_float(my_xcc), __int_as_float(e_sc));
      }
    }
  }
  if (S == 1) return;  // uniform
  // ---- the last split of the sequence to finish merges all S partials
  if (!arrive_last(cnt + b, (uint32_t)S, &sm.last)) return;  // workgroup-uniform
  // 16 heads per round
  if (q_pos) {
    const MergeRope rope = merge_rope(q_pos[b], tid & 31);
    if (S <= 4)
      merge_all_heads<true>(b, H, S, ml, part, out, lse, my_xcc, tid, rope);
    else
      for (int h0 = 0; h0 < H; h0 += 16) merge_splits<true>(b, h0, H, S, ml, part, out, lse, my_xcc, tid, rope);
  } else {
    if (S <= 4)
      merge_all_heads<false>(b, H, S, ml, part, out, lse, my_xcc, tid, MergeRope{});
    else
      for (int h0 = 0; h0 < H; h0 += 16)
        merge_splits<false>(b, h0, H, S, ml, part, out, lse, my_xcc, tid, MergeRope{});
  }
}

// Opt a kernel in to its dynamic LDS size once (thread-safe static init;
// one flag per kernel instantiation).
template <auto Kern>
static bool lds_optin(size_t bytes) {
  static const bool ok =
      hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
  return ok;
}

// Smallest batch for the throughput variant: below it one workgroup per
// sequence leaves too few workgroups, and the split kernel's shorter chain
// wins.
constexpr int kSeqMinBatch = 48;

// row slots: the selected entries, then (from k rounded up to 16 when the
// window holds FP8 records) the window entries; the workspace is sized for
// the rounded count either way
static int attn_slots(int k, int swa_cap, bool w8) { return (w8 ? (k + 15) & ~15 : k) + swa_cap; }
static int attn_splits(int k, int swa_cap) { return (attn_slots(k, swa_cap, true) + kChunk - 1) / kChunk; }

struct AttnWs {
  size_t cnt_off, part_off, ml_off, total;
};

// [counters: kMaxAttnGroups x u32][partials: B*H*S x 512 fp16][(max, sum, xcd, e): B*H*S x 16 B],
// sized for 128-row chunks (the larger S).
static AttnWs attn_ws_layout(int B, int H, int k, int swa_cap) {
  const size_t n = (size_t)B * H * attn_splits(k, swa_cap);
  AttnWs l;
  l.cnt_off = 0;
  l.part_off = (size_t)kMaxAttnGroups * sizeof(uint32_t);
  l.ml_off = l.part_off + ((n * 512 * sizeof(uint16_t) + 255) & ~(size_t)255);
  l.total = l.ml_off + ((n * sizeof(float4) + 255) & ~(size_t)255);
  return l;
}

size_t attn_ws_bytes(int B, int H, int k, int swa_cap) { return attn_ws_layout(B, H, k, swa_cap).total; }


int launch_sparse_attn(const uint16_t* q, int H, const uint8_t* main_codes,
                       const uint8_t* main_scales, int64_t cap, int main_fmt, const int32_t* len,
                       const int32_t* topk, int k, int B, const uint8_t* swa_codes,
                       const uint8_t* swa_scales, int64_t swa_stride, int swa_cap,
                       const int32_t* swa_len, int swa_fmt, float sm_scale, const int64_t* q_pos,
                       uint16_t* out, float* lse_opt, void* ws, hipStream_t st, bool abs_rows, int qps) {
  if (B == 0) return 0;
  // B counts query rows; with qps > 1 query row b reads cache b / qps
  // abs_rows: the index list holds row ids into one pool of cap rows shared
  // by all sequences (no lengths); otherwise positions into sequence b's cap rows
  const int64_t seq_stride = abs_rows ? 0 : cap;
  const bool w8 = swa_fmt == 1 && swa_cap > 0;
  const int nslots = attn_slots(k, swa_cap, w8);
  const int64_t HG = H / 16;
  const int64_t groups = (int64_t)B * HG;
  if (groups > kMaxAttnGroups) return -1;
  // Chunk shape.  A placement unit (a sequence from 8 sequences, else a
  // (sequence, head group)) runs on one XCD of 32 CUs, so what matters is the
  // busiest XCD's workgroup count: 8 waves (128 rows) when it fits the XCD
  // in one round; else 10 waves (160 rows, one workgroup per CU) when those
  // fit; else 8 waves again, two workgroups resident per CU, each hiding the
  // other's latencies.  Measured: 10 waves win at 12 and 16 sequences (12.6
  // against 15.9 us at 16), 8 waves below (10.1 against 10.6 us at 1) and
  // from 20 to 44 (25.7 against 31.3 us at 40).
  const int64_t xunits = B >= 8 ? ((int64_t)B + 7) / 8 * HG : ((int64_t)B * HG + 7) / 8;
  const int64_t x8 = xunits * ((nslots + 127) / 128), x10 = xunits * ((nslots + 159) / 160);
  const bool ten = x8 > 32 && x10 <= 32;
  const int S = ten ? (nslots + 159) / 160 : (nslots + 127) / 128;
  const AttnWs l = attn_ws_layout(B, H, k, swa_cap);
  char* wsb = reinterpret_cast<char*>(ws);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(wsb + l.cnt_off);
  uint16_t* part = reinterpret_cast<uint16_t*>(wsb + l.part_off);
  float4* ml = reinterpret_cast<float4*>(wsb + l.ml_off);
  if (H == 64 && B >= kSeqMinBatch && nslots >= kTRows) {
    // throughput variant: S splits per sequence, enough to give every CU a
    // workgroup, at most one per 128 row slots (the workspace's partials).
    // The grid holds ceil(B / 8) groups of 8 sequences, so S comes from that
    // count: 256 / B splits would overfill the chip where B is not a
    // multiple of 8 (B = 50: 280 workgroups, a second round, 37.9 against
    // 22.8 us).  At most 4 splits: the merge prefetches its next round of
    // partials only then (B = 48: 5 splits 26.8 us, 4 splits 23.1 us).
    const int nch = w8 ? (k + 31) / 32 + (swa_cap + 15) / 16 : (nslots + kTRows - 1) / kTRows;
    int Sq = B >= 256 ? 1 : std::min(4, 32 / (((int)B + 7) / 8));
    Sq = std::min(Sq, std::min(nch, attn_splits(k, swa_cap)));
    const unsigned tgrid = (unsigned)(((B + 7) / 8) * Sq * 8);
    auto tgo = [&](auto kern, bool lds_ok) -> bool {
      if (!lds_ok) return false;
      kern<<<tgrid, 512, sizeof(AttnTSmem), st>>>(q, H, main_codes, main_scales, cap, len, topk, k, swa_codes,
                                                   swa_scales, swa_stride, swa_cap, swa_len, sm_scale, q_pos, B, Sq,
                                                   part, ml, cnt, out, lse_opt, seq_stride, qps);
      return true;
    };
    bool ok;
    if (w8)
      ok = main_fmt == 0 ? tgo(attn_seq_kernel<0, true>, lds_optin<attn_seq_kernel<0, true>>(sizeof(AttnTSmem)))
                         : tgo(attn_seq_kernel<1, true>, lds_optin<attn_seq_kernel<1, true>>(sizeof(AttnTSmem)));
    else
      ok = main_fmt == 0 ? tgo(attn_seq_kernel<0, false>, lds_optin<attn_seq_kernel<0, false>>(sizeof(AttnTSmem)))
                         : tgo(attn_seq_kernel<1, false>, lds_optin<attn_seq_kernel<1, false>>(sizeof(AttnTSmem)));
    if (!ok) return -1;
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int seq_units = B >= 8 ? 1 : 0;
  const int64_t units = seq_units ? B : groups;
  const unsigned grid = (unsigned)(((units + 7) / 8) * (seq_units ? HG : 1) * S * 8);
  auto go = [&](auto kern, int waves, size_t smem, bool lds_ok) -> bool {
    if (!lds_ok) return false;
    kern<<<grid, 64 * waves, smem, st>>>(q, H, main_codes, main_scales, cap, len, topk, k, swa_codes,
                                         swa_scales, swa_stride, swa_cap, swa_len, sm_scale, q_pos, B, S,
                                         part, ml, cnt, out, lse_opt, seq_units, seq_stride, qps);
    return true;
  };
  auto pick = [&](auto fmt_c, auto w8_c) -> bool {
    constexpr int F = decltype(fmt_c)::value;
    constexpr bool W8 = decltype(w8_c)::value;
    if (ten)
      return go(attn_split_kernel<F, 10, W8>, 10, sizeof(AttnSmem<10>),
                lds_optin<attn_split_kernel<F, 10, W8>>(sizeof(AttnSmem<10>)));
    return go(attn_split_kernel<F, 8, W8>, 8, sizeof(AttnSmem<8>),
              lds_optin<attn_split_kernel<F, 8, W8>>(sizeof(AttnSmem<8>)));
  };
  using F0 = std::integral_constant<int, 0>;
  using F1 = std::integral_constant<int, 1>;
  using WN = std::integral_constant<bool, false>;
  using WY = std::integral_constant<bool, true>;
  bool ok;
  if (w8)
    ok = main_fmt == 0 ? pick(F0{}, WY{}) : pick(F1{}, WY{});
  else
    ok = main_fmt == 0 ? pick(F0{}, WN{}) : pick(F1{}, WN{});
  if (!ok) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
