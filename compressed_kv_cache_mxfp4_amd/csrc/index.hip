// index.hip -- hierarchical sparse indexer for CSA2 decode on gfx950.
//
// Full mode [ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析", section 3.3;
// syt-nju.github.io, "为什么读输入只激活 8B", Figure 5; weigao.cc, section 3.2]:
// one scoring pass over every visible indexer-K entry feeds two selections --
// the position top-k (the layer's own attention set) and the block top-n
// (block score = max of its 8 positions, an upper bound) whose expansion is the
// shared candidate pool.  Reindex mode rescores only the pool with the layer's
// own query and takes its own top-k.
//
// score(p) = sum_h w_h * max(0, q_h . K_p), K_p = FP4(E2M1) x E8M0 per 32 dims.
//
// Scoring kernel: streaming, HBM-bound.  Each wave keeps its query's heads in
// registers as bf16 MFMA A-operands and walks 64-entry super-tiles; a lane
// loads 16 B of FP4 codes (32 dims of one entry) plus that group's E8M0 byte,
// which is exactly one B-operand fragment of v_mfma_f32_16x16x32_bf16 after a
// register-level dequantisation (v_cvt_scalef32_pk_bf16_fp4).  The dims of a
// 32-wide K step are permuted identically in A and B, so every load is one
// contiguous 16-byte piece.  ReLU, head weights and the head sum run on the
// accumulators; the 8-entry block maximum is a 3-step lane reduction.
//
// Selection kernel: one 1024-thread workgroup per sequence; keys held in
// registers; an MSB radix search with adaptive bin ranges (2048 LDS bins per
// pass, at most 3 passes) finds the k-th key, then a block scan emits the
// winners in ascending index order with ties resolved to the lower index.
#include "csa2_device.hpp"
#include "csa2.h"
#include "csa2_internal.hpp"

namespace csa2 {

// ======================================================================
// Scoring
// ======================================================================
constexpr int kScoreThreads = 256;
constexpr int kSuperTile = 64;
constexpr int kScoreWaves = 3072;     // full mode: resident waves per launch (3 per SIMD)
constexpr int kScoreWavesPool = 2048;  // pool mode holds more registers (2 per SIMD)

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, true);
}

// Rows of the four 16-entry tiles of one super-tile as seen by lane (g, n):
// entry base + 16t + n of tile t.  Entries past the end map to row 0 (always
// present: the cache holds at least one row), so loads need no branch.
struct ScoreRows {
  int32_t r[4];
  uint32_t ok;  // bit t: entry of tile t exists and is visible
};

// Paged cache, full mode: the rows of the super-tile at `base` through the
// page table.  Its 64 entries share one page (pages hold at least 64
// entries), so one wave-uniform (scalar) table load serves the super-tile.
__device__ __forceinline__ void score_rows_paged(ScoreRows& R, int64_t base, int64_t N, const PageMap& pm,
                                                 int cache, int n) {
  const int tb = __builtin_amdgcn_readfirstlane((int)(base < N ? base >> pm.shift : 0));
  const int32_t pbase = page_base(pm, cache, (int64_t)tb << pm.shift);
  const int32_t mask = (1 << pm.shift) - 1;
  R.ok = 0u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t it = base + 16 * t + n;
    const bool in = it < N;
    R.r[t] = in ? pbase + (int32_t)(it & mask) : 0;
    R.ok |= (in ? 1u : 0u) << t;
  }
}

// Loaded operands of one super-tile: tile t's codes (entry 16t+n, dims
// 32g..32g+31) and the E8M0 byte of that (entry, group).
struct ScoreStage {
  uint4 cw[4];
  uint32_t sb[4];
};

template <bool GATHER>
__device__ __forceinline__ void score_rows(ScoreRows& R, int64_t base, int64_t N, int64_t L,
                                           const int32_t* __restrict__ pool_b, int n) {
  R.ok = 0u;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t it = base + 16 * t + n;
    const bool in = it < N;
    int32_t row;
    if (GATHER) {
      const int32_t p = pool_b[in ? it : 0];
      const bool vis = in && p >= 0 && (int64_t)p < L;
      row = vis ? p : 0;
      R.ok |= (vis ? 1u : 0u) << t;
    } else {
      row = in ? (int32_t)it : 0;
      R.ok |= (in ? 1u : 0u) << t;
    }
    R.r[t] = row;
  }
}

// Byte offsets fit 32 bits (at most CSA2_MAX_CACHE_ROWS rows of 64 B per
// sequence), so loads take a uniform base plus a 32-bit lane offset.
__device__ __forceinline__ void score_load(ScoreStage& S, const ScoreRows& R,
                                           const uint8_t* __restrict__ codes_b,
                                           const uint8_t* __restrict__ scales_b, int g) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t r = (uint32_t)R.r[t];
    S.cw[t] = *reinterpret_cast<const uint4*>(codes_b + (r * 64u + 16u * (uint32_t)g));
    S.sb[t] = scales_b[r * 4u + (uint32_t)g];
  }
}

// Score of entry 16g+n of the super-tile (lane order), before masking.
template <int MT>
__device__ __forceinline__ float score_compute(const ScoreStage& S, const bf16x8 (&A)[MT][4],
                                               const float (&wr)[MT][4]) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const float sop = e8m0_operand(S.sb[t]);
    const uint32_t cw[4] = {S.cw[t].x, S.cw[t].y, S.cw[t].z, S.cw[t].w};
    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 bv = fp4x8_to_bf16(cw[ks], sop);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mt][ks], bv, acc[mt], 0, 0, 0);
    }
    // lane (g, n) holds heads 16mt+4g+i of entry 16t+n
    float p = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p += wr[mt][i] * __int_as_float(max(__float_as_int(acc[mt][i]), 0));
    part[t] = p;
  }
  // Reduce-scatter over the four 16-lane rows: row g ends with tile g's sum.
  const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
  const float s02 = __uint_as_float(a02[0]) + __uint_as_float(a02[1]);
  const float s13 = __uint_as_float(a13[0]) + __uint_as_float(a13[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// FP4 query (both operands MX-FP4, E8M0 per 32 dims): one
// v_mfma_scale_f32_16x16x128_f8f6f4 per (tile, 16 heads) over all 128 dims.
// Lane (g, n) of B is entry 16t+n, dims 32g..32g+31 -- the stage's 16-byte
// code load as it is -- with that block's scale byte; lane (g, i) of A is
// head 16mt+i over the same dims.  D has the bf16 path's layout, so the
// epilogue is the same.
typedef int intx8 __attribute__((ext_vector_type(8)));

template <int MT>
__device__ __forceinline__ float score_compute_q4(const ScoreStage& S, const uint4 (&Aq)[MT],
                                                  const uint32_t (&Asc)[MT], const float (&wr)[MT][4]) {
  float part[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const intx8 bv = {(int)S.cw[t].x, (int)S.cw[t].y, (int)S.cw[t].z, (int)S.cw[t].w, 0, 0, 0, 0};
    floatx4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const intx8 av = {(int)Aq[mt].x, (int)Aq[mt].y, (int)Aq[mt].z, (int)Aq[mt].w, 0, 0, 0, 0};
      acc[mt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          av, bv, floatx4{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, (int)Asc[mt], 0, (int)S.sb[t]);
    }
    float p = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p += wr[mt][i] * __int_as_float(max(__float_as_int(acc[mt][i]), 0));
    part[t] = p;
  }
  const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
  const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
  const float s02 = __uint_as_float(a02[0]) + __uint_as_float(a02[1]);
  const float s13 = __uint_as_float(a13[0]) + __uint_as_float(a13[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float max8_lanes(float v) {
  v = fmaxf(v, __uint_as_float(dpp_mov<0xB1>(__float_as_uint(v), 0u)));   // xor 1
  v = fmaxf(v, __uint_as_float(dpp_mov<0x4E>(__float_as_uint(v), 0u)));   // xor 2
  v = fmaxf(v, __uint_as_float(dpp_mov<0x141>(__float_as_uint(v), 0u)));  // half-row mirror
  return v;
}

// Grid: (workgroups per sequence, B).  Persistent waves: wave j of a
// sequence scores super-tiles j, j + W, j + 2W, ... (W waves per sequence)
// through a ring of kScoreStages operand stages, so kScoreStages - 1
// super-tiles are in flight while one is computed.  With GATHER the items
// are pool[b][i], otherwise positions i; the pool entries of a super-tile
// are read one ring step before its codes.
constexpr int kScoreStages = 2;

template <int MT, bool GATHER, bool Q4 = false, bool PAGED = false, int NS = kScoreStages, int OCC = 2,
          bool WLDS = false>
__global__ __launch_bounds__(kScoreThreads, OCC) void score_kernel(
    const uint8_t* __restrict__ idx_codes, const uint8_t* __restrict__ idx_scales, int64_t cap,
    const int32_t* __restrict__ len, const int32_t* __restrict__ pool,
    const int32_t* __restrict__ pool_len, int pool_cap, const uint16_t* __restrict__ q,
    const float* __restrict__ w, int H, float* __restrict__ scores, int64_t score_stride,
    float* __restrict__ bmax, int64_t bmax_stride, int B, int per_seq,
    const uint8_t* __restrict__ q4_codes, const uint8_t* __restrict__ q4_scales, int qps, PageMap pm,
    int64_t seq_stride) {
  __shared__ __align__(16) uint16_t qs[Q4 ? 8 : 64 * 128];
  __shared__ float ws[64];
  // Grid: per_seq workgroups for each of the B query rows, in one dimension;
  // row b scores cache b / qps (qps queries per cache, e.g. the tokens of a
  // verify block).  Ids run in (cache, walker x, query) order, so the qps
  // queries of a cache walk the same super-tiles side by side and all but
  // the first find them in L2.  When the number of caches is a multiple of
  // 8, cache c's workgroups all get ids congruent to c mod 8, i.e. they run
  // on XCD c mod 8 (with one query per cache, the XCD of the selection
  // workgroup that reads their output next).
  const int id = blockIdx.x;
  const int per_c = per_seq * qps;
  int cb, x, qi;
  if (((B / qps) & 7) == 0) {
    const int r = id >> 3;
    cb = (id & 7) + 8 * (r / per_c);
    x = (r % per_c) / qps;
    qi = r % qps;
  } else {
    cb = id / per_c;
    x = (id % per_c) / qps;
    qi = id % qps;
  }
  const int b = cb * qps + qi;  // query row
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, n = lane & 15;
  const int64_t W = (int64_t)per_seq * 4;
  const int64_t st0 = (int64_t)x * 4 + wave;
  const int64_t step = W * kSuperTile;
  const int64_t base0 = st0 * kSuperTile;
  const int64_t Nmax = GATHER ? (int64_t)pool_cap : cap;  // bound of the item index
  // seq_stride: rows between sequences' caches (0: one pool, physical rows)
  const uint8_t* codes_b = idx_codes + (int64_t)cb * seq_stride * 64;
  const uint8_t* scales_b = idx_scales + (int64_t)cb * seq_stride * 4;
  const int32_t* pool_b = GATHER ? pool + (int64_t)b * pool_cap : nullptr;
  float* scores_b = scores + (int64_t)b * score_stride;

  // The first stages' loads need no length: full mode reads its rows right
  // away (masked later), pool mode reads its pool entries.  They overlap the
  // query staging below, and the lengths are applied after the barrier.
  ScoreRows rows[NS];
  ScoreStage stg[NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    // raw rows: the pool entry itself (-1 past the pool), or the position
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t it = base0 + u * step + 16 * t + n;
      const bool in = it < Nmax;
      if (GATHER)
        rows[u].r[t] = in ? pool_b[it] : -1;
      else
        rows[u].r[t] = in ? (int32_t)it : 0;
    }
    if (PAGED) score_rows_paged(rows[u], base0 + u * step, Nmax, pm, cb, n);
    rows[u].ok = 0u;
  }
  if (!GATHER) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) score_load(stg[u], rows[u], codes_b, scales_b, g);
  }

  // Query heads (zero beyond H; bf16 queries only -- FP4 queries are read
  // straight into their MFMA operands below) and head weights, staged once
  // per workgroup.
  uint4 Aq[MT];
  uint32_t Asc[MT];
  if constexpr (Q4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = 16 * mt + n;
      Aq[mt] = h < H ? *reinterpret_cast<const uint4*>(q4_codes + ((int64_t)b * H + h) * 64 + 16 * g)
                     : make_uint4(0u, 0u, 0u, 0u);
      Asc[mt] = h < H ? q4_scales[((int64_t)b * H + h) * 4 + g] : 127u;
    }
  } else {
    const int h = threadIdx.x >> 2, part = threadIdx.x & 3;  // 64 heads x 4 pieces of 64 B
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = h < H ? *reinterpret_cast<const uint4*>(q + ((int64_t)b * H + h) * 128 + 32 * part + 8 * j)
                   : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&qs[h * 128 + 32 * part + 8 * j]) = v[j];
  }
  if (threadIdx.x < 64) ws[threadIdx.x] = (int)threadIdx.x < H ? w[(int64_t)b * H + threadIdx.x] : 0.0f;
  int64_t L = len ? len[cb] : cap;  // no lengths: pool rows below cap
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int64_t N = L;
  if (GATHER) {
    int64_t pl = pool_len[b];
    N = pl < 0 ? 0 : (pl > pool_cap ? pool_cap : pl);
  }
  __syncthreads();
  if (base0 >= N) return;  // wave-uniform; no barrier follows
  // A operand (bf16 queries): lane (g, m) holds head 16*mt+m, dims 32g+8ks .. +7.
  bf16x8 A[Q4 ? 1 : MT][4];
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if constexpr (!Q4) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        A[mt][ks] = *reinterpret_cast<const bf16x8*>(&qs[(16 * mt + n) * 128 + 32 * g + 8 * ks]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[mt][i] = ws[16 * mt + 4 * g + i];
  }
  const float4* wq = reinterpret_cast<const float4*>(ws) + g;  // heads 16mt+4g .. +3 at wq[4mt]

  // apply the lengths to the early rows (pool mode: entries past pool_len or
  // outside [0, len) are masked and read row 0)
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    rows[u].ok = 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t it = base0 + u * step + 16 * t + n;
      bool vis = it < N;
      if (GATHER) {
        vis = vis && rows[u].r[t] >= 0 && (int64_t)rows[u].r[t] < L;
        rows[u].r[t] = vis ? rows[u].r[t] : 0;
      }
      rows[u].ok |= (vis ? 1u : 0u) << t;
    }
  }
  if (GATHER) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) score_load(stg[u], rows[u], codes_b, scales_b, g);
  }
  const int64_t iters = (N - base0 + step - 1) / step;  // >= 1
  // ring invariant at the top of round r (iteration i = r*NS + u handled by
  // slot u): stages hold iterations i .. i+NS-2, rows[(u+NS-1)%NS] iteration i+NS-1
  for (int64_t i0 = 0; i0 < iters; i0 += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int64_t i = i0 + u;
      const int64_t bs = base0 + i * step;
      const uint32_t ok = rows[u].ok;
      // refill: stage of iteration i+NS-1 (its rows are ready), rows of i+NS
      score_load(stg[(u + NS - 1) % NS], rows[(u + NS - 1) % NS], codes_b, scales_b, g);
      if (PAGED)
        score_rows_paged(rows[u], bs + NS * step, N, pm, cb, n);
      else
        score_rows<GATHER>(rows[u], bs + NS * step, N, L, pool_b, n);
      if (i < iters) {
        if (WLDS) {
          // head weights re-read from LDS each super-tile (keeps 16 VGPRs free)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const float4 v = wq[4 * mt];
            wr[mt][0] = v.x; wr[mt][1] = v.y; wr[mt][2] = v.z; wr[mt][3] = v.w;
          }
        }
        float sc;
        if constexpr (Q4) sc = score_compute_q4<MT>(stg[u], Aq, Asc, wr);
        else sc = score_compute<MT>(stg[u], A, wr);
        const int64_t it = bs + lane;
        const bool mine_ok = (ok >> g) & 1u;
        if (it < N) scores_b[it] = mine_ok ? sc : __uint_as_float(0x7FC00000u);
        // maximum of each group of 8 consecutive items (a cache block, or 8
        // pool entries); a group with no visible item gets NaN (absent)
        const float bm = max8_lanes((it < N && mine_ok) ? sc : -INFINITY);
        if ((lane & 7) == 0 && it < N)
          bmax[(int64_t)b * bmax_stride + (it >> 3)] = bm == -INFINITY ? __uint_as_float(0x7FC00000u) : bm;
      }
    }
  }
}

// ======================================================================
// Selection
// ======================================================================
// One workgroup per sequence.  Keys (monotone uint32 images of the scores)
// sit in registers with wave-contiguous ownership: candidate i lives in wave
// i / (64*E), slot (i / 64) % E, lane i % 64, so loads are coalesced 64-wide
// runs.  The k-th key is found by an MSB radix search whose bin range adapts
// to the keys present (2048 LDS bins per pass, at most 3 passes); the winners
// are emitted in ascending candidate order through wave ballots.  Ordering:
// larger key first, equal keys to the lower candidate index.  Wave-level
// reductions and scans use DPP (row shifts, mirrors, row broadcasts).

// Reduce within each 16-lane row (every lane of the row gets the row's value).
template <class Op>
__device__ __forceinline__ uint32_t row_reduce(uint32_t v, Op op) {
  v = op(v, dpp_mov<0xB1>(v, 0u));   // quad_perm [1,0,3,2]
  v = op(v, dpp_mov<0x4E>(v, 0u));   // quad_perm [2,3,0,1]
  v = op(v, dpp_mov<0x141>(v, 0u));  // row_half_mirror
  v = op(v, dpp_mov<0x140>(v, 0u));  // row_mirror
  return v;
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
  v = row_reduce(v, op);
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp_mov<0x111>(x, 0u);       // row_shr:1
  x += dpp_mov<0x112>(x, 0u);       // row_shr:2
  x += dpp_mov<0x114>(x, 0u);       // row_shr:4
  x += dpp_mov<0x118>(x, 0u);       // row_shr:8
  x += dpp_mov<0x142, 0xa>(x, 0u);  // row_bcast:15 into rows 1 and 3
  x += dpp_mov<0x143, 0xc>(x, 0u);  // row_bcast:31 into rows 2 and 3
  return x;
}

struct __align__(16) SelScratch {
  uint32_t hist[2][2048];  // double-buffered: one is cleared while the other is filled
  uint32_t wred[3][16];
  uint32_t bc[4];
};

// Candidates that survive the prefilter, in ascending candidate order: key,
// candidate index and one caller value each (96 KB of LDS: the prefilter's
// sample rank leaves about 1.5 k + n / 64 survivors, 4096 for k = 2048 of
// 65,536, so half the capacity is margin).  Compaction pays
// off from 32 keys per thread (more than 32K candidates): it adds one pass
// over every key (about 10 instructions per key, 16 SIMD cycles each with
// 16 waves on 4 SIMDs) and saves the radix passes' and the emission's per-key
// work; measured on the Full call's block selection, 65,536 blocks per
// sequence: 34.5 -> 29.3 us and 35.5 -> 27.8 us for the two selections, and
// at 16,384 blocks 0.5-0.9 us slower, so it is not used there.
constexpr int kCompactCap = 8192;
constexpr int kCompactMinEpt = 32;
struct __align__(16) SelCompact {
  uint32_t key[kCompactCap];
  int32_t idx[kCompactCap];
  uint32_t side[kCompactCap];
};

// No per-candidate caller value.
struct NoSide {
  __device__ uint32_t operator()(int, int) const { return 0u; }
};

// Keys of a compaction buffer.
struct KeysFromLdsC {
  const uint32_t* p;
  __device__ uint32_t key(int i) const { return p[i]; }
};

// float -> uint32 key with the same order; NaN (absent) -> 0; -0 -> +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f != f) return 0u;
  if (f == 0.0f) return 0x80000000u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int EPT>
struct KeyRegs {
  uint32_t r[EPT > 0 ? EPT : 1];
};

// Candidate of slot j for this thread.
template <int NT, int EPT>
__device__ __forceinline__ int sel_index(int n, int j) {
  const int E = EPT > 0 ? EPT : (n + NT - 1) / NT;
  return (threadIdx.x >> 6) * 64 * E + 64 * j + (threadIdx.x & 63);
}

template <int NT, int EPT, class Src>
__device__ __forceinline__ void load_keys(KeyRegs<EPT>& K, const Src& src, int n) {
  if constexpr (EPT > 0) {
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int i = sel_index<NT, EPT>(n, j);
      K.r[j] = i < n ? src.key(i) : 0u;
    }
  }
}

// Keys of a float array in two steps, so that the loads need not wait for
// the candidate count: load_raw reads every slot below n_alloc (the array's
// allocated length), finish_keys then turns slots below n into keys and the
// rest into 0 (absent).
// Slot j of a thread is base + 64 j (sel_index), so bounds are tested as
// 64 j < n - base against one per-thread remainder: no per-slot index stays live.
template <int NT, int EPT>
__device__ __forceinline__ void load_raw(KeyRegs<EPT>& K, const float* p, int n_alloc) {
  const int base = sel_index<NT, EPT>(0, 0);
  const int rem = n_alloc - base;
  const float* pb = p + base;
#pragma unroll
  for (int j = 0; j < EPT; ++j) K.r[j] = 64 * j < rem ? __float_as_uint(pb[64 * j]) : 0x7FC00000u;
}

template <int NT, int EPT>
__device__ __forceinline__ void finish_keys(KeyRegs<EPT>& K, int n) {
  const int rem = n - sel_index<NT, EPT>(0, 0);
#pragma unroll
  for (int j = 0; j < EPT; ++j) K.r[j] = 64 * j < rem ? float_key(__uint_as_float(K.r[j])) : 0u;
}

// Sum of the per-wave values w[0 .. wave-1] (wave < 16): lane v < wave reads
// w[v], then one 16-lane reduction.  One LDS round trip, a few VALU ops.
__device__ __forceinline__ uint32_t wave_prefix(const uint32_t* w, int wave) {
  const int lane = threadIdx.x & 63;
  uint32_t v = lane < wave ? w[lane] : 0u;
  v = row_reduce(v, [](uint32_t x, uint32_t y) { return x + y; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
}

// Bin of histogram h (2048 bins, ascending key order; bins past the used
// range are zero) that holds the need-th largest counted key.  Thread t scans
// bins 2047-TB*t .. 2048-TB*(t+1) in descending order; a block scan of the
// per-thread sums locates the owner, which writes (bin, count above the bin)
// to bc[0..1].  Ends with a barrier, so bc is visible on return.
template <int NT>
__device__ __forceinline__ void find_bin_from_top(const uint32_t* h, SelScratch& sh, uint32_t need) {
  constexpr int TB = 2048 / NT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int top = 2047 - TB * t;
  uint32_t hb[TB];
  uint32_t s = 0u;
#pragma unroll
  for (int j = 0; j < TB; ++j) {
    hb[j] = h[top - j];
    s += hb[j];
  }
  const uint32_t incl = wave_incl_scan(s);
  if (lane == 63) sh.wred[0][wave] = incl;
  __syncthreads();
  uint32_t excl = incl - s + wave_prefix(sh.wred[0], wave);
  if (excl < need && need <= excl + s) {
    uint32_t acc = excl;
#pragma unroll
    for (int j = 0; j < TB; ++j) {
      if (acc < need && need <= acc + hb[j]) {
        sh.bc[0] = (uint32_t)(top - j);
        sh.bc[1] = acc;
        sh.bc[2] = hb[j];
      }
      acc += hb[j];
    }
  }
  __syncthreads();
}

// Top-k of the n candidates (key 0 = absent): calls emit(i, rank, key, side)
// for the winners in ascending i, rank = 0, 1, ..., with side = side_fn(j, i)
// evaluated by the thread whose key slot j holds candidate i; returns
// min(k, #present).
//
// PREF: when the candidates far outnumber k, a sample (one key per thread)
// first bounds the k-th key from below: T0 = lower edge of the histogram bin
// holding a sample rank with a wide margin.  If at least k keys are >= T0
// (checked exactly), the radix search only histograms keys in [T0, max];
// otherwise it searches the full range.  With a compaction buffer cp and at
// most kCompactCap keys >= T0, those keys are first copied to cp in
// ascending candidate order and the search and the emission run over them
// alone (a few keys per thread instead of all n).  Either way the result is
// exact and the same.
template <int NT, int EPT, bool PREF, class Src, class Emit, class Side = NoSide>
__device__ __forceinline__ int select_core(const KeyRegs<EPT>& K, const Src& src, int n, int k, SelScratch& sh,
                           Emit emit, SelCompact* cp = nullptr, Side side_fn = Side{}) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 16, "per-wave partials hold at most 16 waves");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int E = EPT > 0 ? EPT : (n + NT - 1) / NT;
  auto KEY = [&](int j) -> uint32_t {
    if constexpr (EPT > 0) {
      return K.r[j];
    } else {
      const int i = sel_index<NT, EPT>(n, j);
      return i < n ? src.key(i) : 0u;
    }
  };
  constexpr int UNR = EPT > 0 ? EPT : 1;

  // both histogram buffers start cleared; the barrier after the reduction
  // below orders these stores before any histogram update
  for (int i = t; i < 2 * 2048; i += NT) (&sh.hist[0][0])[i] = 0u;
  uint32_t cnt = 0u, mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll UNR
  for (int j = 0; j < E; ++j) {
    const uint32_t kk = KEY(j);
    cnt += kk ? 1u : 0u;
    mn = kk ? min(mn, kk) : mn;
    mx = max(mx, kk);
  }
  cnt = wave_reduce(cnt, [](uint32_t a, uint32_t b) { return a + b; });
  mn = wave_reduce(mn, [](uint32_t a, uint32_t b) { return min(a, b); });
  mx = wave_reduce(mx, [](uint32_t a, uint32_t b) { return max(a, b); });
  if (lane == 0) {
    sh.wred[0][wave] = cnt;
    sh.wred[1][wave] = mn;
    sh.wred[2][wave] = mx;
  }
  __syncthreads();
  cnt = sh.wred[0][0];
  mn = sh.wred[1][0];
  mx = sh.wred[2][0];
#pragma unroll
  for (int v = 1; v < NW; ++v) {
    cnt += sh.wred[0][v];
    mn = min(mn, sh.wred[1][v]);
    mx = max(mx, sh.wred[2][v]);
  }
  // No barrier here: the prefilter and every pass synchronise before they
  // write wred; only the emission can follow directly (synced == false).
  const uint32_t target = min((uint32_t)k, cnt);
  bool synced = false;  // a barrier has passed since the partials were read
  if (target == 0u) {
    __syncthreads();  // every wave has read the partials before a later call reuses them
    return 0;
  }

  uint32_t lo = mn, hi = mx, above = 0u, T;
  bool take_all_eq = false;
  int buf = 0;  // histogram buffer of the next pass
  if constexpr (PREF) {
    if (lo != hi && cnt > 4096u && cnt >= 8u * target) {
      const uint32_t span = hi - lo;
      const int nbits = 32 - __clz((int)span);
      const int shift = nbits > 11 ? nbits - 11 : 0;
      const uint32_t smp = KEY(0);
      if (smp) atomicAdd(&sh.hist[0][(smp - lo) >> shift], 1u);
      if (t == 0) sh.bc[0] = 0xFFFFFFFFu;
      __syncthreads();
      synced = true;
      // sample rank: 1.5x the expected share of the k winners, plus 16
      const uint32_t r = min((uint32_t)NT, 16u + (uint32_t)((3ull * target * NT + 2ull * cnt - 1) / (2ull * cnt)));
      find_bin_from_top<NT>(sh.hist[0], sh, r);
      const uint32_t tb = sh.bc[0];
      const uint32_t T0 = tb == 0xFFFFFFFFu ? lo : lo + (tb << shift);
      for (int i = t; i < 2048; i += NT) sh.hist[0][i] = 0u;
      uint32_t c0 = 0u;
  #pragma unroll UNR
      for (int j = 0; j < E; ++j) c0 += (uint32_t)__popcll(__ballot(KEY(j) >= T0));
      // wred[0]: read by find_bin above before its last barrier; the emission
      // below writes only wred[1] and wred[2]
      if (lane == 0) sh.wred[0][wave] = c0;
      __syncthreads();
      c0 = 0u;
  #pragma unroll
      for (int v = 0; v < NW; ++v) c0 += sh.wred[0][v];
      if (c0 >= target) {
        lo = T0;
        if (cp != nullptr && c0 <= (uint32_t)kCompactCap) {
          // survivors to cp in candidate order: earlier waves' counts, then
          // slot by slot through the wave's ballots
          const uint64_t below = (1ull << lane) - 1ull;
          uint32_t off = wave_prefix(sh.wred[0], wave);
  #pragma unroll UNR
          for (int j = 0; j < E; ++j) {
            const uint32_t kk = KEY(j);
            const bool sv = kk >= T0;
            const uint64_t m = __ballot(sv);
            if (sv) {
              const uint32_t at = off + (uint32_t)__popcll(m & below);
              const int i = sel_index<NT, EPT>(n, j);
              cp->key[at] = kk;
              cp->idx[at] = i;
              cp->side[at] = side_fn(j, i);
            }
            off += (uint32_t)__popcll(m);
            if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
          }
          __syncthreads();  // also: every wave has read wred[0]
          constexpr int EC = kCompactCap / NT;
          KeysFromLdsC csrc{cp->key};
          KeyRegs<EC> kc;
          load_keys<NT, EC>(kc, csrc, (int)c0);
          return select_core<NT, EC, false>(kc, csrc, (int)c0, k, sh, [&](int ci, int r, uint32_t key, uint32_t) {
            emit(cp->idx[ci], r, key, cp->side[ci]);
          });
        }
      }
    }
  }
  for (;;) {
    if (lo == hi) {
      T = lo;
      break;
    }
    const uint32_t span = hi - lo;
    const int nbits = 32 - __clz((int)span);
    const int shift = nbits > 11 ? nbits - 11 : 0;
    uint32_t* h = sh.hist[buf];
#pragma unroll UNR
    for (int j = 0; j < E; ++j) {
      const uint32_t kk = KEY(j);
      if (kk >= lo && kk <= hi) atomicAdd(&h[(kk - lo) >> shift], 1u);
      if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // bound register pressure at large E
    }
    uint32_t* hn = sh.hist[buf ^ 1];
    for (int i = t; i < 2048; i += NT) hn[i] = 0u;  // the next pass's buffer
    __syncthreads();
    synced = true;
    find_bin_from_top<NT>(h, sh, target - above);
    const uint32_t tb = sh.bc[0], gt = sh.bc[1], in_bin = sh.bc[2];
    if (target - above - gt == in_bin) {
      // every key of the boundary bin is selected: take all keys >= its lower edge
      T = lo + (tb << shift);
      take_all_eq = true;
      break;
    }
    above += gt;
    const uint32_t nlo = lo + (tb << shift);
    const uint32_t width = (1u << shift) - 1u;
    hi = (hi - nlo < width) ? hi : nlo + width;
    lo = nlo;
    buf ^= 1;
    if (shift == 0) {
      T = lo;
      break;
    }
  }
  const uint32_t need_eq = take_all_eq ? 0xFFFFFFFFu : target - above;

  // per-wave counts above / equal to the threshold, then ordered emission
  uint32_t wgt = 0u, weq = 0u;
#pragma unroll UNR
  for (int j = 0; j < E; ++j) {
    const uint32_t kk = KEY(j);
    wgt += (uint32_t)__popcll(__ballot(kk > T));
    weq += (uint32_t)__popcll(__ballot(kk == T));
  }
  if (!synced) __syncthreads();  // workgroup-uniform: all keys were equal
  if (lane == 0) {
    sh.wred[1][wave] = wgt;
    sh.wred[2][wave] = weq;
  }
  __syncthreads();
  // Earlier waves' totals: G (keys above T) and E (keys equal to T).  The
  // equal keys are taken in index order up to need_eq, so the earlier waves
  // emitted G + min(E, need_eq).  Lanes 0-15 sum wred[1], lanes 16-31 wred[2].
  uint32_t eq_pref, out_pref;
  {
    uint32_t v = lane < wave ? sh.wred[1][lane] : ((lane >= 16 && lane - 16 < wave) ? sh.wred[2][lane - 16] : 0u);
    v = row_reduce(v, [](uint32_t x, uint32_t y) { return x + y; });
    const uint32_t G = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    eq_pref = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    out_pref = G + min(eq_pref, need_eq);
  }
  const uint64_t below = (1ull << lane) - 1ull;
  const int ibase = sel_index<NT, EPT>(n, 0);  // slot j holds candidate ibase + 64 j
  uint32_t r_sel = out_pref, r_eq = eq_pref;
#pragma unroll UNR
  for (int j = 0; j < E; ++j) {
    const uint32_t kk = KEY(j);
    bool sel = kk > T;
    const uint64_t eqb = __ballot(kk == T);
    if (eqb) {  // wave-uniform: rare, only around the threshold
      const uint32_t eq_rank = r_eq + (uint32_t)__popcll(eqb & below);
      sel = sel || (kk == T && eq_rank < need_eq);
      r_eq += (uint32_t)__popcll(eqb);
    }
    const uint64_t selb = __ballot(sel);
    if (selb) {  // wave-uniform
      if (sel) emit(ibase + 64 * j, (int)(r_sel + (uint32_t)__popcll(selb & below)), kk, side_fn(j, ibase + 64 * j));
      r_sel += (uint32_t)__popcll(selb);
    }
    if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  return (int)target;
}

struct KeysFromArray {
  const float* p;
  __device__ uint32_t key(int i) const { return float_key(p[i]); }
};

struct KeysFromLds {
  const uint32_t* p;
  __device__ uint32_t key(int i) const { return p[i]; }
};

constexpr int kBlock = 8;

// Items of candidate groups: candidate i is item grp[i/8]*8 + i%8.
struct KeysFromGroups {
  const float* scores;
  const int32_t* grp;
  __device__ int item(int i) const { return grp[i >> 3] * kBlock + (i & 7); }
  __device__ uint32_t key(int i) const { return float_key(scores[item(i)]); }
};

// Group selection prunes item selection exactly: take contiguous groups of
// items (8 positions of a cache block, or 8 consecutive pool entries) ranked
// by (group max desc, group index asc).  Every group ranked ahead of the
// group of an item p holds a distinct item ranked ahead of p (its maximum:
// larger, or equal and at a lower index), so an item of rank < k lies in a
// group of rank < k.  The item top-k is therefore exact over the items of the
// top-k groups.

// Number of items covered by the first ng selected groups (the last group of
// the n items may be partial).
__device__ __forceinline__ int group_items(const int32_t* grp, int ng, int n_items) {
  int nc = ng * kBlock;
  const int last = (n_items + kBlock - 1) / kBlock - 1;
  if (ng > 0 && grp[ng - 1] == last) nc -= last * kBlock + kBlock - n_items;
  return nc;
}

// Full-mode selection for one sequence (grid = B; with a pool 2B, one
// workgroup running 1 and one running 2-3, side by side):
//  1. block top-n_blocks -> pool (ascending positions), with the sampled
//     prefilter (2048 of 16,384 blocks at 128K);
//  2. block top-k -> candidate blocks, among the pool blocks when
//     n_blocks >= k (the top-k blocks are among the top-n_blocks blocks),
//     otherwise among all blocks;
//  3. position top-k over the positions of those blocks (group pruning).
template <int NT, int EPT_B, int EPT_C, int EPT_P>
__global__ __launch_bounds__(NT) void select_full_kernel(
    const float* __restrict__ scores, int64_t sstride, const float* __restrict__ bmax,
    int64_t bstride, const int32_t* __restrict__ len, int64_t cap, int k, int n_blocks,
    int32_t* __restrict__ topk, int32_t* __restrict__ pool, int32_t* __restrict__ pool_len, int qps,
    PageMap pm, int32_t* __restrict__ topk_rows, int32_t* __restrict__ pool_rows, int B, int split) {
  __shared__ SelScratch sh;
  __shared__ int32_t blk[CSA2_POOL_BLOCKS];
  __shared__ uint32_t blkkey[CSA2_POOL_BLOCKS];
  __shared__ int32_t cblk[CSA2_MAX_TOPK];
  __shared__ SelCompact cpt;
  // split: two workgroups per sequence, one per selection (role 0 the pool,
  // role 1 the top-k, which then takes its blocks from all blocks -- the
  // same set, the pool being the top blocks by the same key), so the two
  // run side by side.  Both get ids congruent to b mod 8 when B is a
  // multiple of 8: the XCD whose L2 holds the sequence's scores.
  int b, role;
  if (!split) {
    b = blockIdx.x;
    role = -1;  // both
  } else if ((B & 7) == 0) {
    b = (int)(blockIdx.x & 7) + 8 * (int)(blockIdx.x >> 4);
    role = (blockIdx.x >> 3) & 1;
  } else {
    b = blockIdx.x >> 1;
    role = blockIdx.x & 1;
  }
  KeysFromArray bsrc{bmax + (int64_t)b * bstride};
  KeyRegs<EPT_B> kb;
  if constexpr (EPT_B > 0) load_raw<NT, EPT_B>(kb, bsrc.p, (int)bstride);  // overlaps the length load
  int64_t L = len[b / qps];  // row b scores cache b / qps
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nb = (int)((L + kBlock - 1) / kBlock);
  const float* sc = scores + (int64_t)b * sstride;
  int32_t* tk = topk + (int64_t)b * k;
  // paged cache: the selections' physical rows too (row ids for the gathers)
  int32_t* tkr = topk_rows ? topk_rows + (int64_t)b * k : nullptr;
  if constexpr (EPT_B > 0) finish_keys<NT, EPT_B>(kb, nb);
  int ncb;
  if (n_blocks > 0 && role != 1) {
    const int nsel = select_core<NT, EPT_B, true>(
        kb, bsrc, nb, n_blocks, sh,
        [&](int i, int r, uint32_t key, uint32_t) {
          blk[r] = i;
          blkkey[r] = key;
        },
        EPT_B >= kCompactMinEpt ? &cpt : nullptr);
    const int pl = group_items(blk, nsel, (int)L);
    int32_t* pb = pool + (int64_t)b * n_blocks * kBlock;
    // a thread writes whole groups (8 entries: two 16-byte stores when the
    // caller's buffer allows it)
    const bool vec = (reinterpret_cast<uintptr_t>(pb) & 15u) == 0u;
    int32_t* pbr = pool_rows ? pool_rows + (int64_t)b * n_blocks * kBlock : nullptr;
    for (int gi = threadIdx.x; gi < n_blocks; gi += NT) {
      const int base = gi * kBlock;
      const int p0 = gi < nsel ? blk[gi] * kBlock : 0;
      int e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = base + j < pl ? p0 + j : -1;
      if (vec) {
        int4* dst = reinterpret_cast<int4*>(pb + base);
        dst[0] = make_int4(e[0], e[1], e[2], e[3]);
        dst[1] = make_int4(e[4], e[5], e[6], e[7]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[base + j] = e[j];
      }
      if (pbr) {
        // a block of 8 never straddles a page (pages hold >= 64 entries)
        const int32_t r0 = base < pl ? page_row(pm, b / qps, p0) : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) pbr[base + j] = e[j] >= 0 ? r0 + j : -1;
      }
    }
    if (threadIdx.x == 0) pool_len[b] = pl;
  }
  if (role == 0) return;  // workgroup-uniform: the pool was this workgroup's part
  if (n_blocks >= k && role == -1) {
    // top-k among the selected pool blocks (keys kept in LDS, ascending blocks)
    const int nsel = min(n_blocks, nb);
    KeysFromLds csrc{blkkey};
    KeyRegs<EPT_C> kc;
    load_keys<NT, EPT_C>(kc, csrc, nsel);
    ncb = select_core<NT, EPT_C, false>(kc, csrc, nsel, k, sh,
                                        [&](int i, int r, uint32_t, uint32_t) { cblk[r] = blk[i]; });
  } else {
    ncb = select_core<NT, EPT_B, true>(kb, bsrc, nb, k, sh, [&](int i, int r, uint32_t, uint32_t) { cblk[r] = i; },
                                       EPT_B >= kCompactMinEpt ? &cpt : nullptr);
  }
  const int nc = group_items(cblk, ncb, (int)L);
  KeysFromGroups psrc{sc, cblk};
  KeyRegs<EPT_P> kp;
  load_keys<NT, EPT_P>(kp, psrc, nc);
  const int cnt = select_core<NT, EPT_P, true>(
      kp, psrc, nc, k, sh,
      [&](int i, int r, uint32_t, uint32_t) {
        tk[r] = psrc.item(i);
        if (tkr) tkr[r] = page_row(pm, b / qps, psrc.item(i));
      },
      EPT_P >= kCompactMinEpt ? &cpt : nullptr);
  for (int i = cnt + threadIdx.x; i < k; i += NT) {
    tk[i] = -1;
    if (tkr) tkr[i] = -1;
  }
}

// Reindex selection: top-k of the pool scores (NaN = masked entry) through
// the top-k groups of 8 consecutive pool entries (group maxima written by the
// scoring kernel).  The pool positions of the candidates are loaded with
// their keys, so emission needs no further memory round trip.
template <int NT, int EPT_G, int EPT_P>
__global__ __launch_bounds__(NT) void select_pool_kernel(
    const float* __restrict__ pool_scores, const float* __restrict__ gmax,
    const int32_t* __restrict__ pool, const int32_t* __restrict__ pool_len, int pool_cap, int k,
    int32_t* __restrict__ topk, const int32_t* __restrict__ pool_rows, int32_t* __restrict__ topk_rows) {
  __shared__ SelScratch sh;
  __shared__ int32_t cgrp[CSA2_MAX_TOPK];
  const int b = blockIdx.x;
  const int ngs = (pool_cap + kBlock - 1) / kBlock;
  KeysFromArray gsrc{gmax + (int64_t)b * ngs};
  KeyRegs<EPT_G> kg;
  load_raw<NT, EPT_G>(kg, gsrc.p, ngs);  // overlaps the pool length load
  int n = pool_len[b];
  n = n < 0 ? 0 : (n > pool_cap ? pool_cap : n);
  const int ng = (n + kBlock - 1) / kBlock;
  const int32_t* pb = pool + (int64_t)b * pool_cap;
  int32_t* tk = topk + (int64_t)b * k;
  // the selections' physical rows too, when the pool has them
  const int32_t* pbr = pool_rows ? pool_rows + (int64_t)b * pool_cap : nullptr;
  int32_t* tkr = topk_rows ? topk_rows + (int64_t)b * k : nullptr;
  finish_keys<NT, EPT_G>(kg, ng);
  const int ncg = select_core<NT, EPT_G, false>(kg, gsrc, ng, k, sh, [&](int i, int r, uint32_t, uint32_t) { cgrp[r] = i; });
  const int nc = group_items(cgrp, ncg, n);
  KeysFromGroups psrc{pool_scores + (int64_t)b * pool_cap, cgrp};
  KeyRegs<EPT_P> kp;
  int32_t pos[EPT_P > 0 ? EPT_P : 1];
  if constexpr (EPT_P > 0) {
#pragma unroll
    for (int j = 0; j < EPT_P; ++j) {
      const int i = sel_index<NT, EPT_P>(nc, j);
      const int item = i < nc ? psrc.item(i) : 0;
      kp.r[j] = i < nc ? float_key(psrc.scores[item]) : 0u;
      pos[j] = i < nc ? pb[item] : -1;
    }
  }
  const int cnt = select_core<NT, EPT_P, true>(
      kp, psrc, nc, k, sh,
      [&](int i, int r, uint32_t, uint32_t side) {
        if constexpr (EPT_P > 0) tk[r] = (int32_t)side; else tk[r] = pb[psrc.item(i)];
        if (tkr) tkr[r] = pbr[psrc.item(i)];
      },
      nullptr, [&](int j, int) -> uint32_t {  // at most 16 keys per thread here: no compaction
        if constexpr (EPT_P > 0) return (uint32_t)pos[j]; else return 0u;
      });
  for (int i = cnt + threadIdx.x; i < k; i += NT) {
    tk[i] = -1;
    if (tkr) tkr[i] = -1;
  }
}

// ======================================================================
// Host launchers
// ======================================================================
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

IndexFullWs index_full_ws_layout(int B, int64_t cap, int block) {
  IndexFullWs l;
  l.scores_off = 0;
  l.bmax_off = align256((size_t)B * (size_t)cap * 4);
  const int64_t nb = (cap + block - 1) / block;
  l.total = l.bmax_off + align256((size_t)B * (size_t)nb * 4);
  return l;
}

// q4_codes == nullptr: bf16 queries `q`; otherwise FP4 queries (codes, scales).
template <bool GATHER>
static void launch_score(int MT, int per_seq, int B, hipStream_t st, const uint8_t* ic, const uint8_t* is,
                         int64_t cap, const int32_t* len, const int32_t* pool,
                         const int32_t* pool_len, int pool_cap, const uint16_t* q, const uint8_t* q4c,
                         const uint8_t* q4s, const float* w, int H, float* scores, int64_t sstride,
                         float* bmax, int64_t bstride, int qps = 1, PageMap pm = PageMap{nullptr, 0, 0, 0},
                         int64_t seq_stride = -1) {
  const dim3 grid((unsigned)per_seq * (unsigned)B);
  if (seq_stride < 0) seq_stride = cap;
#define CSA2_SCORE(MT_, Q4_, PG_) \
  score_kernel<MT_, GATHER, Q4_, PG_><<<grid, kScoreThreads, 0, st>>>(ic, is, cap, len, pool, pool_len, pool_cap, q, \
                                                                      w, H, scores, sstride, bmax, bstride, B, per_seq, \
                                                                      q4c, q4s, qps, pm, seq_stride)
  if (!GATHER && pm.table) {
    if (q4c) {
      if (MT == 1) CSA2_SCORE(1, true, true); else if (MT == 2) CSA2_SCORE(2, true, true); else CSA2_SCORE(4, true, true);
    } else {
      if (MT == 1) CSA2_SCORE(1, false, true); else if (MT == 2) CSA2_SCORE(2, false, true); else CSA2_SCORE(4, false, true);
    }
  } else if (q4c) {
    if (MT == 1) CSA2_SCORE(1, true, false); else if (MT == 2) CSA2_SCORE(2, true, false); else CSA2_SCORE(4, true, false);
  } else {
    if (MT == 1) CSA2_SCORE(1, false, false); else if (MT == 2) CSA2_SCORE(2, false, false); else CSA2_SCORE(4, false, false);
  }
#undef CSA2_SCORE
}

// Workgroups per sequence for `items` scored entries: enough resident waves
// to cover the chip, never more than one super-tile per wave.  When the
// resident target binds, the count rounds down: the waves walk their
// super-tiles with a grid stride, and a launch even slightly over the target
// would run its last workgroups as a second, nearly empty round (80 query
// rows of 16,384 pool entries: 7 workgroups a row is 2,240 waves against
// 2,048 resident, 6 is 1,920).
static unsigned score_wgs(int64_t items, int B, int target_waves) {
  const int64_t tiles = (items + kSuperTile - 1) / kSuperTile;
  int64_t waves = target_waves / (B > 0 ? B : 1);
  if (waves < 4) waves = 4;
  const int64_t wgs = waves >= tiles ? (tiles + 3) / 4 : waves / 4;
  return (unsigned)(wgs > 0 ? wgs : 1);
}

int launch_index_full_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int B, const uint16_t* q, const uint8_t* q4c,
                            const uint8_t* q4s, const float* w, int H, int block, float* scores_opt, void* ws,
                            hipStream_t st, int qps, PageMap pm) {
  if (B == 0) return 0;
  const IndexFullWs l = index_full_ws_layout(B, cap, block);
  float* scores = scores_opt ? scores_opt : reinterpret_cast<float*>((char*)ws + l.scores_off);
  float* bmax = reinterpret_cast<float*>((char*)ws + l.bmax_off);
  const int64_t nbk = (cap + block - 1) / block;
  const int MT = (H + 15) / 16;
  const int per_seq = (int)score_wgs(cap, B, kScoreWaves);
  if (cap > 0)
    launch_score<false>(MT, per_seq, B, st, idx_codes, idx_scales, cap, len, nullptr, nullptr, 0, q, q4c,
                        q4s, w, H, scores, cap, bmax, nbk, qps, pm, pm.table ? 0 : cap);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_index_full(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                      const int32_t* len, int B, const uint16_t* q, const uint8_t* q4c,
                      const uint8_t* q4s, const float* w, int H, int k,
                      int block, int n_blocks, int32_t* topk, int32_t* pool, int32_t* pool_len,
                      float* scores_opt, void* ws, hipStream_t st, int qps, PageMap pm, int32_t* topk_rows,
                      int32_t* pool_rows) {
  if (B == 0) return 0;
  if (launch_index_full_score(idx_codes, idx_scales, cap, len, B, q, q4c, q4s, w, H, block, scores_opt, ws, st,
                              qps, pm) != 0)
    return -1;
  return launch_index_full_select(cap, len, B, k, block, n_blocks, topk, pool, pool_len, scores_opt, ws, st, qps,
                                  pm, topk_rows, pool_rows);
}

int launch_index_full_select(int64_t cap, const int32_t* len, int B, int k, int block, int n_blocks,
                             int32_t* topk, int32_t* pool, int32_t* pool_len, const float* scores_opt, void* ws,
                             hipStream_t st, int qps, PageMap pm, int32_t* topk_rows, int32_t* pool_rows) {
  if (B == 0) return 0;
  const IndexFullWs l = index_full_ws_layout(B, cap, block);
  const float* scores = scores_opt ? scores_opt : reinterpret_cast<const float*>((char*)ws + l.scores_off);
  const float* bmax = reinterpret_cast<const float*>((char*)ws + l.bmax_off);
  const int64_t nbk = (cap + block - 1) / block;
  const bool kbig = k > 512;
  // the pool and the top-k as two workgroups per sequence when there is a pool
  const bool split = n_blocks > 0;
  // keys per thread: all blocks (EB), the pool blocks (2), candidate positions (EP)
#define CSA2_SELFULL(EB, EP) \
  select_full_kernel<1024, EB, 2, EP><<<B * (split ? 2 : 1), 1024, 0, st>>>(scores, cap, bmax, nbk, len, cap, k, \
                                                         n_blocks, topk, pool, pool_len, qps, pm, topk_rows, \
                                                         pool_rows, B, split ? 1 : 0)
  if (nbk <= 4 * 1024) {
    if (kbig) CSA2_SELFULL(4, 16); else CSA2_SELFULL(4, 4);
  } else if (nbk <= 16 * 1024) {
    if (kbig) CSA2_SELFULL(16, 16); else CSA2_SELFULL(16, 4);
  } else if (nbk <= 32 * 1024) {
    if (kbig) CSA2_SELFULL(32, 16); else CSA2_SELFULL(32, 4);
  } else if (nbk <= 64 * 1024) {
    if (kbig) CSA2_SELFULL(64, 16); else CSA2_SELFULL(64, 4);
  } else {
    if (kbig) CSA2_SELFULL(0, 16); else CSA2_SELFULL(0, 4);
  }
#undef CSA2_SELFULL
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Workspace of the Reindex call: pool scores (unless the caller supplies the
// buffer), then the maxima of groups of 8 pool entries.
struct IndexPoolWs {
  size_t scores_off, gmax_off, total;
};

static IndexPoolWs index_pool_ws_layout(int B, int pool_cap) {
  IndexPoolWs l;
  l.scores_off = 0;
  l.gmax_off = align256((size_t)B * (size_t)pool_cap * 4);
  l.total = l.gmax_off + align256((size_t)B * (size_t)((pool_cap + kBlock - 1) / kBlock) * 4);
  return l;
}

size_t index_pool_ws_bytes(int B, int pool_cap) { return index_pool_ws_layout(B, pool_cap).total; }

int launch_index_pool_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int B, const int32_t* pool, const int32_t* pool_len,
                            int pool_cap, const uint16_t* q, const uint8_t* q4c, const uint8_t* q4s,
                            const float* w, int H, float* pool_scores_opt, void* ws, hipStream_t st,
                            const int32_t* pool_rows, int qps) {
  // B counts query rows; with qps > 1 row b rescores its own pool over cache b / qps
  if (B == 0) return 0;
  const IndexPoolWs l = index_pool_ws_layout(B, pool_cap);
  float* ps = pool_scores_opt ? pool_scores_opt : reinterpret_cast<float*>((char*)ws + l.scores_off);
  float* gmax = reinterpret_cast<float*>((char*)ws + l.gmax_off);
  const int64_t ngs = (pool_cap + kBlock - 1) / kBlock;
  const int MT = (H + 15) / 16;
  const int per_seq = (int)score_wgs(pool_cap, B, kScoreWavesPool);
  if (pool_cap > 0)
    // with physical pool rows: gather from one pool of cap rows, no lengths
    launch_score<true>(MT, per_seq, B, st, idx_codes, idx_scales, cap, pool_rows ? nullptr : len,
                       pool_rows ? pool_rows : pool, pool_len, pool_cap, q, q4c, q4s, w, H, ps, pool_cap, gmax, ngs,
                       qps, PageMap{nullptr, 0, 0, 0}, pool_rows ? 0 : cap);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_index_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                      const int32_t* len, int B, const int32_t* pool, const int32_t* pool_len,
                      int pool_cap, const uint16_t* q, const uint8_t* q4c, const uint8_t* q4s,
                      const float* w, int H, int k,
                      int32_t* topk, float* pool_scores_opt, void* ws, hipStream_t st,
                      const int32_t* pool_rows, int32_t* topk_rows, int qps) {
  if (B == 0) return 0;
  if (launch_index_pool_score(idx_codes, idx_scales, cap, len, B, pool, pool_len, pool_cap, q, q4c, q4s, w, H,
                              pool_scores_opt, ws, st, pool_rows, qps) != 0)
    return -1;
  return launch_index_pool_select(B, pool, pool_len, pool_cap, k, topk, pool_scores_opt, ws, st, pool_rows,
                                  topk_rows);
}

int launch_index_pool_select(int B, const int32_t* pool, const int32_t* pool_len, int pool_cap, int k,
                             int32_t* topk, const float* pool_scores_opt, void* ws, hipStream_t st,
                             const int32_t* pool_rows, int32_t* topk_rows) {
  if (B == 0) return 0;
  const IndexPoolWs l = index_pool_ws_layout(B, pool_cap);
  const float* ps = pool_scores_opt ? pool_scores_opt : reinterpret_cast<const float*>((char*)ws + l.scores_off);
  const float* gmax = reinterpret_cast<const float*>((char*)ws + l.gmax_off);
  // keys per thread: groups (<= 2048 -> 2), candidate positions (8 per selected group)
  if (k <= 512)
    select_pool_kernel<1024, 2, 4><<<B, 1024, 0, st>>>(ps, gmax, pool, pool_len, pool_cap, k, topk, pool_rows,
                                                       topk_rows);
  else
    select_pool_kernel<1024, 2, 16><<<B, 1024, 0, st>>>(ps, gmax, pool, pool_len, pool_cap, k, topk, pool_rows,
                                                        topk_rows);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa2
