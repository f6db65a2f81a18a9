// csa2_internal.hpp -- host-side launchers shared between the translation
// units of libcsa2 (not part of the public C ABI).  Each returns 0 on success
// and -1 when a launch failed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Page map of a paged cache: entry i of sequence c lives at physical row
// (table[c * max_pages + (i >> shift)] << shift) + (i & (2^shift - 1)) of one
// pool of n_pages << shift rows shared by all sequences.  table == nullptr:
// not paged.  A table entry outside [0, n_pages) is clamped into the pool,
// so a stale entry reads a wrong row of the pool, never outside it.
struct PageMap {
  const int32_t* table;
  int shift;
  int max_pages;
  int32_t n_pages;
};

__device__ __forceinline__ int32_t page_base(const PageMap& pm, int c, int64_t i) {
  int32_t pg = pm.table[(int64_t)c * pm.max_pages + (i >> pm.shift)];
  pg = pg < 0 ? 0 : (pg >= pm.n_pages ? pm.n_pages - 1 : pg);
  return pg << pm.shift;
}

__device__ __forceinline__ int32_t page_row(const PageMap& pm, int c, int64_t i) {
  return page_base(pm, c, i) + (int32_t)(i & ((1 << pm.shift) - 1));
}


int launch_quantize(const float* x, int64_t rows, int dim, int group, int fmt, uint8_t* codes,
                    uint8_t* scales, hipStream_t st);

int launch_cache_write(const uint16_t* latent, const uint16_t* gate, int64_t T, int m,
                       const float* gamma, float eps, const float* w_idx, int main_fmt,
                       const int64_t* rope_pos, uint8_t* main_codes, uint8_t* main_scales,
                       uint8_t* idx_codes, uint8_t* idx_scales, hipStream_t st);

size_t append_state_bytes(int B);
int launch_cache_append(const uint16_t* latent, const uint16_t* gate, int B, int m, const float* gamma,
                        float eps, const float* w_idx, int main_fmt, int rope, uint8_t* main_codes,
                        uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales, int64_t cap,
                        int32_t* len, void* state, hipStream_t st,
                        PageMap pm = PageMap{nullptr, 0, 0, 0});

// Workspace layout of the indexer calls (bytes, 256-aligned pieces).
struct IndexFullWs {
  size_t scores_off, bmax_off, total;
};
IndexFullWs index_full_ws_layout(int B, int64_t cap, int block);

// q4c/q4s: FP4 queries (codes [B][H][64], E8M0 scales [B][H][4]); when
// q4c is NULL the bf16 queries q are used.
int launch_index_full(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                      const int32_t* len, int B, const uint16_t* q, const uint8_t* q4c,
                      const uint8_t* q4s, const float* w, int H, int k,
                      int block, int n_blocks, int32_t* topk, int32_t* pool, int32_t* pool_len,
                      float* scores_opt, void* ws, hipStream_t st, int qps = 1,
                      PageMap pm = PageMap{nullptr, 0, 0, 0}, int32_t* topk_rows = nullptr,
                      int32_t* pool_rows = nullptr);

// The two phases of launch_index_full: scoring (scores and block maxima into
// the workspace, or the scores into scores_opt) and the selections from them.
int launch_index_full_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int B, const uint16_t* q, const uint8_t* q4c,
                            const uint8_t* q4s, const float* w, int H, int block, float* scores_opt, void* ws,
                            hipStream_t st, int qps = 1, PageMap pm = PageMap{nullptr, 0, 0, 0});
int launch_index_full_select(int64_t cap, const int32_t* len, int B, int k, int block, int n_blocks,
                             int32_t* topk, int32_t* pool, int32_t* pool_len, const float* scores_opt, void* ws,
                             hipStream_t st, int qps = 1, PageMap pm = PageMap{nullptr, 0, 0, 0},
                             int32_t* topk_rows = nullptr, int32_t* pool_rows = nullptr);

size_t index_pool_ws_bytes(int B, int pool_cap);

// The two phases of launch_index_pool.
int launch_index_pool_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int B, const int32_t* pool, const int32_t* pool_len,
                            int pool_cap, const uint16_t* q, const uint8_t* q4c, const uint8_t* q4s,
                            const float* w, int H, float* pool_scores_opt, void* ws, hipStream_t st,
                            const int32_t* pool_rows = nullptr, int qps = 1);
int launch_index_pool_select(int B, const int32_t* pool, const int32_t* pool_len, int pool_cap, int k,
                             int32_t* topk, const float* pool_scores_opt, void* ws, hipStream_t st,
                             const int32_t* pool_rows = nullptr, int32_t* topk_rows = nullptr);

int launch_index_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                      const int32_t* len, int B, const int32_t* pool, const int32_t* pool_len,
                      int pool_cap, const uint16_t* q, const uint8_t* q4c, const uint8_t* q4s,
                      const float* w, int H, int k,
                      int32_t* topk, float* pool_scores_opt, void* ws, hipStream_t st,
                      const int32_t* pool_rows = nullptr, int32_t* topk_rows = nullptr, int qps = 1);

size_t attn_ws_bytes(int B, int H, int k, int swa_cap);

int launch_sparse_attn(const uint16_t* q, int H, const uint8_t* main_codes,
                       const uint8_t* main_scales, int64_t cap, int main_fmt, const int32_t* len,
                       const int32_t* topk, int k, int B, const uint8_t* swa_codes,
                       const uint8_t* swa_scales, int64_t swa_stride, int swa_cap,
                       const int32_t* swa_len, int swa_fmt, float sm_scale, const int64_t* q_pos,
                       uint16_t* out, float* lse_opt, void* ws, hipStream_t st, bool abs_rows = false,
                       int qps = 1);
int launch_window_write(const uint16_t* latent, int B, int n, const float* gamma, float eps, int rope,
                        const int64_t* pos0, int W, uint8_t* data, uint8_t* scales, int32_t* swa_len,
                        hipStream_t st);

}  // namespace csa2
