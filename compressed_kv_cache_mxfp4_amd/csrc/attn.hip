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
// One workgroup (8 waves) per (sequence, group of 16 heads).  A decode call is
// bound by memory latency (two dependent round trips: the index list, then
// the rows), so every row load of the workgroup is issued before any math:
// up to 640 rows (a super-chunk) sit in registers as raw FP4 (72 bytes per
// lane).  Two passes per super-chunk: pass 1 computes every logit from the
// registers (independent MFMA chains per 128-row chunk) and reduces the exact
// max and sum once; pass 2 re-dequantises each chunk into LDS for P.R.  Longer
// selections run several super-chunks joined by an online-softmax rescale.
//  * Q.R^T: wave w takes rows 16w..16w+15 of each 128-row chunk.  Lane (g, m) holds 64
//    code bytes of row m (dims 128g..128g+127) and their 8 scale bytes and
//    dequantises them straight into the A operand of v_mfma_f32_16x16x32_bf16:
//    K step ks covers dims 128g+8ks..+7 in lane group g, and the query
//    fragments (B operand, from an LDS copy of the 16 queries) use the same
//    permutation.  The bf16 rows are also stored row-major in LDS.
//  * P.R: wave w takes dims 64w..64w+63 for the 16 heads.  P comes from LDS;
//    the row-major R tile is read column-wise with the gfx950 transpose read
//    (ds_read_b64_tr_b16): within a 16-lane group, source lane a+4j points at
//    R[r0+j][d0+4a] and lane n receives R[r0..r0+3][d0+n], i.e. four K slots
//    of the MFMA B operand.
#include "csa2_device.hpp"
#include "csa2_internal.hpp"

namespace csa2 {

constexpr int kChunk = 128;            // rows per chunk (8 waves x 16)
constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kPrefetch = 5;           // chunks whose rows are loaded up front
constexpr int kRLd = 520;              // R row stride in bf16 (padded)
constexpr int kPLd = 136;              // P row stride in bf16 (padded)

typedef short shortx4 __attribute__((ext_vector_type(4)));

struct AttnSmem {
  uint16_t R[kChunk * kRLd];
  uint16_t Q[16 * kRLd];
  uint16_t P[16 * kPLd];
  float red_m[kAttnWaves][16];
  float red_l[kAttnWaves][16];
};

// Eight E2M1 values of one code dword -> bf16x8 (exact).
template <int FMT>
__device__ __forceinline__ bf16x8 dequant8(uint32_t codes, uint32_t sbyte) {
  if (FMT == 0) {
    return fp4x8_to_bf16(codes, e8m0_operand(sbyte));
  } else {
    const float s = e4m3_value(sbyte);
    float f[8];
    fp4x8_to_f32(codes, f);
    uint4 u;
    u.x = f32_to_bf16_bits(f[0] * s) | (f32_to_bf16_bits(f[1] * s) << 16);
    u.y = f32_to_bf16_bits(f[2] * s) | (f32_to_bf16_bits(f[3] * s) << 16);
    u.z = f32_to_bf16_bits(f[4] * s) | (f32_to_bf16_bits(f[5] * s) << 16);
    u.w = f32_to_bf16_bits(f[6] * s) | (f32_to_bf16_bits(f[7] * s) << 16);
    return __builtin_bit_cast(bf16x8, u);
  }
}

struct RowFetch {
  uint4 c[4];   // 64 code bytes: dims 128g .. 128g+127 of the lane's row
  uint2 s;      // 8 scale bytes: groups 8g .. 8g+7
  uint32_t ok;  // row exists and is visible
};

struct RowSrc {
  const uint8_t* codes;
  const uint8_t* scales;
  uint32_t ok;
};

// Where row slot `slot` of sequence b lives (selected entry or window entry);
// `p` is the already-loaded index-list entry for slots below k.
__device__ __forceinline__ RowSrc locate_row(int slot, int32_t p, int nslots, int b, int k,
                                             int64_t L, int SL, int64_t cap, int64_t swa_stride,
                                             const uint8_t* __restrict__ main_codes,
                                             const uint8_t* __restrict__ main_scales,
                                             const uint8_t* __restrict__ swa_codes,
                                             const uint8_t* __restrict__ swa_scales) {
  RowSrc r{nullptr, nullptr, 0u};
  if (slot < k) {
    if (p >= 0 && (int64_t)p < L) {
      r.codes = main_codes + ((int64_t)b * cap + p) * 256;
      r.scales = main_scales + ((int64_t)b * cap + p) * 32;
      r.ok = 1u;
    }
  } else if (slot < nslots) {
    const int rr = slot - k;
    if (rr < SL) {
      r.codes = swa_codes + ((int64_t)b * swa_stride + rr) * 256;
      r.scales = swa_scales + ((int64_t)b * swa_stride + rr) * 32;
      r.ok = 1u;
    }
  }
  return r;
}

__device__ __forceinline__ void fetch_row(RowFetch& f, const RowSrc& r, int g) {
  if (r.ok) {
    const uint4* c4 = reinterpret_cast<const uint4*>(r.codes + 64 * g);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.c[j] = c4[j];
    f.s = *reinterpret_cast<const uint2*>(r.scales + 8 * g);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.c[j] = make_uint4(0u, 0u, 0u, 0u);
    f.s = make_uint2(0u, 0u);
  }
  f.ok = r.ok;
}

// Dequantise the 16 K steps of one lane's row slice (dims 128g..128g+127).
template <int FMT>
__device__ __forceinline__ bf16x8 row_step(const RowFetch& f, int ks) {
  const uint4 c4 = f.c[ks >> 2];
  const uint32_t cwd = (ks & 3) == 0 ? c4.x : ((ks & 3) == 1 ? c4.y : ((ks & 3) == 2 ? c4.z : c4.w));
  const uint32_t sbyte = (((ks >> 1) < 4 ? f.s.x : f.s.y) >> (8 * ((ks >> 1) & 3))) & 0xFFu;
  return dequant8<FMT>(cwd, sbyte);
}

template <int FMT>
__global__ __launch_bounds__(kAttnThreads, 1) void attn_kernel(
    const uint16_t* __restrict__ q, int H, const uint8_t* __restrict__ main_codes,
    const uint8_t* __restrict__ main_scales, int64_t cap, const int32_t* __restrict__ len,
    const int32_t* __restrict__ topk, int k, const uint8_t* __restrict__ swa_codes,
    const uint8_t* __restrict__ swa_scales, int64_t swa_stride, int swa_cap,
    const int32_t* __restrict__ swa_len, float sm_scale, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem& sm = *reinterpret_cast<AttnSmem*>(smem_raw);
  const int hg = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, n = lane & 15;
  const int nslots = k + swa_cap;
  int64_t L = len ? len[b] : 0;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int SL = swa_len ? swa_len[b] : 0;
  SL = SL < 0 ? 0 : (SL > swa_cap ? swa_cap : SL);
  const int ta = n & 3, tj = n >> 2;

  // running statistics of heads 4g+i (O side) across super-chunks
  float Mrun[4], Lrun[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { Mrun[i] = -INFINITY; Lrun[i] = 0.f; }
  float MrunP = -INFINITY;  // the same running max for head n (P side)
  floatx4 O[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Super-chunks of kPrefetch*kChunk row slots (one for k + window <= 640).
  for (int s0 = 0; s0 < nslots; s0 += kPrefetch * kChunk) {
    const int nch = min(kPrefetch, (nslots - s0 + kChunk - 1) / kChunk);
    // ---- prologue: two round trips (index-list entries, then every row load)
    int32_t pidx[kPrefetch];
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc) {
      const int slot = s0 + cc * kChunk + 16 * w + n;
      const int32_t v = k > 0 ? topk[(int64_t)b * k + min(slot, k - 1)] : -1;
      pidx[cc] = slot < k ? v : -1;
    }
    uint4 qv[2];
    if (s0 == 0) {
      const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)b * H + 16 * hg) * 512);
#pragma unroll
      for (int j = 0; j < 2; ++j) qv[j] = qp[tid + kAttnThreads * j];  // 16 heads x 64 pieces
    }
    RowFetch rows[kPrefetch];
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc) {
      const RowSrc src = locate_row(s0 + cc * kChunk + 16 * w + n, pidx[cc], nslots, b, k, L, SL,
                                    cap, swa_stride, main_codes, main_scales, swa_codes, swa_scales);
      fetch_row(rows[cc], src, g);
    }
    if (s0 == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int e = tid + kAttnThreads * j;
        *reinterpret_cast<uint4*>(&sm.Q[(e >> 6) * kRLd + 8 * (e & 63)]) = qv[j];
      }
    }
    __syncthreads();

    // ---- pass 1: logits of the wave's 16 rows of every chunk (independent MFMA chains)
    floatx4 sacc[kPrefetch];
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc) sacc[cc] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 qf = *reinterpret_cast<const bf16x8*>(&sm.Q[n * kRLd + 128 * g + 8 * ks]);
#pragma unroll
      for (int cc = 0; cc < kPrefetch; ++cc) {
        if (cc < nch)
          sacc[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(row_step<FMT>(rows[cc], ks), qf, sacc[cc], 0, 0, 0);
      }
    }
    float x[kPrefetch][4];
    float mw = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc) {
      const uint64_t vmask = __ballot(rows[cc].ok != 0u);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = cc < nch && ((vmask >> (4 * g + i)) & 1ull);
        x[cc][i] = ok ? sacc[cc][i] * sm_scale : -INFINITY;
        mw = fmaxf(mw, x[cc][i]);
      }
    }
    mw = fmaxf(mw, shfl_xor_f(mw, 16));
    mw = fmaxf(mw, shfl_xor_f(mw, 32));
    if (g == 0) sm.red_m[w][n] = mw;
    __syncthreads();
    float Msc = sm.red_m[0][n];
#pragma unroll
    for (int v = 1; v < kAttnWaves; ++v) Msc = fmaxf(Msc, sm.red_m[v][n]);
    const float MnewP = fmaxf(MrunP, Msc);
    MrunP = MnewP;
    float lw = 0.f;
    uint32_t pb[kPrefetch][4];
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (MnewP == -INFINITY) ? 0.0f : __expf(x[cc][i] - MnewP);
        pb[cc][i] = f32_to_bf16_bits(p);
        lw += p;
      }
    lw += shfl_xor_f(lw, 16);
    lw += shfl_xor_f(lw, 32);
    if (g == 0) sm.red_l[w][n] = lw;

    // ---- pass 2: per chunk, R (re-dequantised) and P to LDS, then O += P.R
#pragma unroll
    for (int cc = 0; cc < kPrefetch; ++cc) {
      if (cc >= nch) break;  // workgroup-uniform
      uint16_t* rrow = &sm.R[(16 * w + n) * kRLd + 128 * g];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) *reinterpret_cast<bf16x8*>(rrow + 8 * ks) = row_step<FMT>(rows[cc], ks);
      *reinterpret_cast<uint2*>(&sm.P[n * kPLd + 16 * w + 4 * g]) =
          make_uint2(pb[cc][0] | (pb[cc][1] << 16), pb[cc][2] | (pb[cc][3] << 16));
      __syncthreads();
      if (cc == 0) {
        // rescale the running output of heads 4g+i to this super-chunk's max
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int hh = 4 * g + i;
          float m2 = sm.red_m[0][hh];
          float l2 = sm.red_l[0][hh];
#pragma unroll
          for (int v = 1; v < kAttnWaves; ++v) {
            m2 = fmaxf(m2, sm.red_m[v][hh]);
            l2 += sm.red_l[v][hh];
          }
          const float mn = fmaxf(Mrun[i], m2);
          const float alpha = (Mrun[i] == -INFINITY) ? 0.0f : __expf(Mrun[i] - mn);
          Lrun[i] = Lrun[i] * alpha + l2;
          Mrun[i] = mn;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) O[nt][i] *= alpha;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&sm.P[n * kPLd + 32 * ks + 8 * g]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int col = 64 * w + 16 * nt + 4 * ta;
          const int r0 = 32 * ks + 8 * g + tj;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)(&sm.R[r0 * kRLd + col]));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) shortx4*)(&sm.R[(r0 + 4) * kRLd + col]));
          shortx8 bv;
          bv[0] = lo[0]; bv[1] = lo[1]; bv[2] = lo[2]; bv[3] = lo[3];
          bv[4] = hi[0]; bv[5] = hi[1]; bv[6] = hi[2]; bv[7] = hi[3];
          O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, bv), O[nt], 0, 0, 0);
        }
      }
      __syncthreads();
    }
  }

  const int h0 = 16 * hg;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * g + i;
    const float inv = Lrun[i] > 0.f ? 1.0f / Lrun[i] : 0.0f;
    uint16_t* orow = out + ((int64_t)b * H + h0 + hh) * 512 + 64 * w + n;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) orow[16 * nt] = (uint16_t)f32_to_bf16_bits(O[nt][i] * inv);
    if (lse && w == 0 && n == 0)
      lse[(int64_t)b * H + h0 + hh] = Lrun[i] > 0.f ? Mrun[i] + logf(Lrun[i]) : -INFINITY;
  }
}

size_t attn_ws_bytes(int B, int H, int k, int swa_cap) {
  (void)B; (void)H; (void)k; (void)swa_cap;
  return 256;  // no scratch is used; a token buffer keeps the interface stable
}

int launch_sparse_attn(const uint16_t* q, int H, const uint8_t* main_codes,
                       const uint8_t* main_scales, int64_t cap, int main_fmt, const int32_t* len,
                       const int32_t* topk, int k, int B, const uint8_t* swa_codes,
                       const uint8_t* swa_scales, int64_t swa_stride, int swa_cap,
                       const int32_t* swa_len, float sm_scale, uint16_t* out, float* lse_opt,
                       void* ws, hipStream_t st) {
  (void)ws;
  if (B == 0) return 0;
  const size_t smem = sizeof(AttnSmem);
  static bool attr_done[2] = {false, false};
  dim3 grid((unsigned)(H / 16), (unsigned)B);
  if (main_fmt == 0) {
    if (!attr_done[0]) {
      hipFuncSetAttribute((const void*)attn_kernel<0>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      attr_done[0] = true;
    }
    attn_kernel<0><<<grid, kAttnThreads, smem, st>>>(q, H, main_codes, main_scales, cap, len, topk, k, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, sm_scale, out, lse_opt);
  } else {
    if (!attr_done[1]) {
      hipFuncSetAttribute((const void*)attn_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
      attr_done[1] = true;
    }
    attn_kernel<1><<<grid, kAttnThreads, smem, st>>>(q, H, main_codes, main_scales, cap, len, topk, k, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, sm_scale, out, lse_opt);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
