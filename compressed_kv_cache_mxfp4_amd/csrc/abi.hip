// abi.hip -- the extern "C" boundary of libcsa2 (declared in include/csa2.h).
// Host-side validation happens here, before any launch; kernels live in
// quant.hip, index.hip and attn.hip.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa2.h"
#include "csa2_internal.hpp"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline int launched(int rc) { return rc == 0 ? CSA2_OK : CSA2_ERR_HIP; }
inline bool valid_fmt(int f) { return f == CSA2_SCALE_E8M0 || f == CSA2_SCALE_E4M3; }
inline bool valid_index_heads(int H) { return H == 8 || H == 16 || H == 32 || H == 64; }

// Argument checks shared by the attention entry points (CSA2_OK: launch).
int check_attn(const uint16_t* q, int32_t H, const uint8_t* main_codes, const uint8_t* main_scales,
               int64_t n_rows, int64_t max_rows, int32_t main_fmt, bool need_len, const int32_t* len,
               const int32_t* sel, int32_t k, int32_t B, const uint8_t* swa_codes, const uint8_t* swa_scales,
               int64_t swa_stride, int32_t swa_cap, const int32_t* swa_len, int32_t swa_fmt, float sm_scale,
               const int64_t* q_pos, const uint16_t* out) {
  if (B < 0 || n_rows < 0 || n_rows > max_rows) return CSA2_ERR_SHAPE;
  if (k < 0 || k > CSA2_MAX_TOPK || swa_cap < 0 || swa_cap > CSA2_SWA) return CSA2_ERR_SHAPE;
  if (H < 16 || H > 64 || H % 16 != 0) return CSA2_ERR_UNSUPPORTED;
  if ((int64_t)B * (H / 16) > CSA2_ATTN_MAX_GROUPS) return CSA2_ERR_SHAPE;
  if (!valid_fmt(main_fmt)) return CSA2_ERR_UNSUPPORTED;
  if (swa_fmt != CSA2_SWA_MAIN && swa_fmt != CSA2_SWA_FP8) return CSA2_ERR_UNSUPPORTED;
  if (k + swa_cap == 0) return CSA2_ERR_SHAPE;
  if (!(sm_scale == sm_scale) || sm_scale == INFINITY || sm_scale == -INFINITY) return CSA2_ERR_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!q || !out) return CSA2_ERR_NULL;
  if (k > 0 && (!main_codes || !main_scales || (need_len && !len) || !sel)) return CSA2_ERR_NULL;
  if (swa_cap > 0 && (!swa_codes || !swa_scales || !swa_len)) return CSA2_ERR_NULL;
  if (swa_cap > 0 && swa_stride < swa_cap) return CSA2_ERR_SHAPE;
  if (!aligned16(q) || (main_codes && !aligned16(main_codes)) || (swa_codes && !aligned16(swa_codes)) ||
      (reinterpret_cast<uintptr_t>(q_pos) & 7u) ||
      (swa_fmt == CSA2_SWA_FP8 && (reinterpret_cast<uintptr_t>(swa_scales) & 7u)))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

// ---- library-held attention scratch for csa2_sparse_attn_decode_noalloc.
// Each GPU holds one copy of `scratch` for the life of the process.  In host
// code the name is only a stand-in for the device symbol: its device address
// is taken once per device with hipGetSymbolAddress, and only that address is
// ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[CSA2_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
int g_scratch_rc[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The scratch address on the current device (nullptr on failure, with the
// status in *rc).  The first call on a device also clears the completion
// counters with a fill kernel on `st` (every attention call leaves them zero
// afterwards).
void* device_scratch(hipStream_t st, int* rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = CSA2_ERR_HIP;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [&] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      g_scratch_rc[dev] = CSA2_ERR_HIP;
      return;
    }
    constexpr int words = CSA2_ATTN_WS_COUNTER_BYTES / 4;
    zero_words_kernel<<<(words + 255) / 256, 256, 0, st>>>(reinterpret_cast<uint32_t*>(ptr), words);
    if (hipGetLastError() != hipSuccess) {
      g_scratch_rc[dev] = CSA2_ERR_HIP;
      return;
    }
    g_scratch_ptr[dev] = ptr;
    g_scratch_rc[dev] = CSA2_OK;
  });
  *rc = g_scratch_rc[dev];
  return *rc == CSA2_OK ? g_scratch_ptr[dev] : nullptr;
}

}  // namespace

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "null pointer argument";
    case CSA2_ERR_SHAPE: return "size argument out of range or inconsistent";
    case CSA2_ERR_ALIGN: return "pointer not 16-byte aligned";
    case CSA2_ERR_UNSUPPORTED: return "unsupported configuration";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch failure";
    case CSA2_ERR_SCRATCH: return "problem larger than the library's fixed attention scratch";
    default: return "unknown status";
  }
}

const char* csa2_version(void) { return "csa2 0.1 gfx950"; }

int csa2_quantize_fp4(const float* x, int64_t rows, int32_t dim, int32_t group, int32_t fmt,
                      uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || dim <= 0 || dim > 4096) return CSA2_ERR_SHAPE;
  if (group != 16 && group != 32) return CSA2_ERR_SHAPE;
  if (dim % group != 0) return CSA2_ERR_SHAPE;
  if (!valid_fmt(fmt)) return CSA2_ERR_UNSUPPORTED;
  if (rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_ERR_NULL;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 1u)) return CSA2_ERR_ALIGN;
  return launched(csa2::launch_quantize(x, rows, dim, group, fmt, codes, scales, as_stream(stream)));
}

int csa2_cache_write(const uint16_t* latent, const uint16_t* gate, int64_t T, int32_t m,
                     const float* gamma, float eps, const float* w_idx, int32_t main_fmt,
                     const int64_t* rope_pos, uint8_t* main_codes, uint8_t* main_scales,
                     uint8_t* idx_codes, uint8_t* idx_scales, void* stream) {
  if (T < 0 || m < 1 || m > 8 || T % m != 0) return CSA2_ERR_SHAPE;
  if (!valid_fmt(main_fmt)) return CSA2_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f)) return CSA2_ERR_SHAPE;
  if (T == 0) return CSA2_OK;
  if (!latent || (m > 1 && !gate) || !w_idx || !main_codes || !main_scales || !idx_codes || !idx_scales)
    return CSA2_ERR_NULL;
  if (!aligned16(latent) || (m > 1 && !aligned16(gate)) || !aligned16(main_codes) ||
      !aligned16(idx_codes) || !aligned16(w_idx) || (reinterpret_cast<uintptr_t>(rope_pos) & 7u))
    return CSA2_ERR_ALIGN;
  return launched(csa2::launch_cache_write(latent, gate, T, m, gamma, eps, w_idx, main_fmt, rope_pos,
                                           main_codes, main_scales, idx_codes, idx_scales,
                                           as_stream(stream)));
}

size_t csa2_append_state_bytes(int32_t B) { return B <= 0 ? 0 : csa2::append_state_bytes(B); }

int csa2_cache_append(const uint16_t* latent, const uint16_t* gate, int32_t B, int32_t m,
                      const float* gamma, float eps, const float* w_idx, int32_t main_fmt, int32_t rope,
                      uint8_t* main_codes, uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales,
                      int64_t cap, int32_t* len, void* state, void* stream) {
  if (B < 0 || m < 1 || m > 2 || cap < 1 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (!valid_fmt(main_fmt)) return CSA2_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f)) return CSA2_ERR_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!latent || (m == 2 && (!gate || !state)) || !w_idx || !main_codes || !main_scales || !idx_codes ||
      !idx_scales || !len)
    return CSA2_ERR_NULL;
  if (!aligned16(latent) || (m == 2 && (!aligned16(gate) || !aligned16(state))) || !aligned16(main_codes) ||
      !aligned16(idx_codes) || (reinterpret_cast<uintptr_t>(w_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(len) & 3u))
    return CSA2_ERR_ALIGN;
  return launched(csa2::launch_cache_append(latent, gate, B, m, gamma, eps, w_idx, main_fmt, rope ? 1 : 0,
                                            main_codes, main_scales, idx_codes, idx_scales, cap, len, state,
                                            as_stream(stream)));
}

int csa2_window_write(const uint16_t* latent, int32_t B, int32_t n, const float* gamma, float eps,
                      int32_t rope, const int64_t* pos0, int32_t W, uint8_t* win_data,
                      uint8_t* win_scales, int32_t* swa_len, void* stream) {
  if (B < 0 || n < 0 || W < 1 || W > CSA2_SWA) return CSA2_ERR_SHAPE;
  if (!(eps >= 0.0f)) return CSA2_ERR_SHAPE;
  if (B == 0 || n == 0) return CSA2_OK;
  if (!latent || !pos0 || !win_data || !win_scales || !swa_len) return CSA2_ERR_NULL;
  if (!aligned16(latent) || !aligned16(win_data) || (reinterpret_cast<uintptr_t>(win_scales) & 7u) ||
      (reinterpret_cast<uintptr_t>(pos0) & 7u) || (reinterpret_cast<uintptr_t>(swa_len) & 3u) ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u))
    return CSA2_ERR_ALIGN;
  return launched(csa2::launch_window_write(latent, B, n, gamma, eps, rope ? 1 : 0, pos0, W, win_data,
                                            win_scales, swa_len, as_stream(stream)));
}

size_t csa2_index_full_workspace(int32_t B, int64_t cap, int32_t k, int32_t block,
                                 int32_t n_blocks) {
  (void)k;
  (void)n_blocks;
  if (B <= 0 || cap <= 0 || block != CSA2_BLOCK) return 0;
  return csa2::index_full_ws_layout(B, cap, block).total;
}

int csa2_index_full(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                    const int32_t* len, int32_t B, const uint16_t* q, const float* w, int32_t H,
                    int32_t k, int32_t block, int32_t n_blocks, int32_t* topk, int32_t* pool,
                    int32_t* pool_len, float* scores_opt, void* ws, size_t ws_bytes,
                    void* stream) {
  if (B < 0 || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !q || !w || !topk) return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_len)) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_workspace(B, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full(idx_codes, idx_scales, cap, len, B, q, nullptr, nullptr, w, H,
                                          k, block, n_blocks, topk, pool, pool_len, scores_opt, ws,
                                          as_stream(stream)));
}

int csa2_index_full_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                          int32_t B, const uint16_t* q, const float* w, int32_t H, int32_t block, float* scores_opt,
                          void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !q || !w) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_workspace(B, cap, 1, block, 0)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full_score(idx_codes, idx_scales, cap, len, B, q, nullptr, nullptr, w, H, block,
                                                scores_opt, ws, as_stream(stream)));
}

int csa2_index_full_select(int64_t cap, const int32_t* len, int32_t B, int32_t k, int32_t block, int32_t n_blocks,
                           int32_t* topk, int32_t* pool, int32_t* pool_len, const float* scores_opt, void* ws,
                           size_t ws_bytes, void* stream) {
  if (B < 0 || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!len || !topk) return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_len)) return CSA2_ERR_NULL;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_workspace(B, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full_select(cap, len, B, k, block, n_blocks, topk, pool, pool_len, scores_opt,
                                                 ws, as_stream(stream)));
}

size_t csa2_index_full_mq_workspace(int32_t B, int32_t Q, int64_t cap, int32_t k, int32_t block,
                                    int32_t n_blocks) {
  if (Q < 1 || Q > CSA2_MAX_QUERIES_PER_SEQ || B <= 0 || (int64_t)B * Q > INT32_MAX) return 0;
  return csa2_index_full_workspace(B * Q, cap, k, block, n_blocks);
}

int csa2_index_full_mq(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                       const int32_t* len, int32_t B, int32_t Q, const uint16_t* q, const float* w,
                       int32_t H, int32_t k, int32_t block, int32_t n_blocks, int32_t* topk,
                       int32_t* pool, int32_t* pool_len, float* scores_opt, void* ws, size_t ws_bytes,
                       void* stream) {
  if (Q < 1 || Q > CSA2_MAX_QUERIES_PER_SEQ) return CSA2_ERR_SHAPE;
  if (B < 0 || (int64_t)B * Q > INT32_MAX || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !q || !w || !topk) return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_len)) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_mq_workspace(B, Q, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full(idx_codes, idx_scales, cap, len, B * Q, q, nullptr, nullptr, w, H,
                                          k, block, n_blocks, topk, pool, pool_len, scores_opt, ws,
                                          as_stream(stream), Q));
}

int csa2_index_full_mq_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int32_t B, int32_t Q, const uint8_t* q_codes,
                            const uint8_t* q_scales, const float* w, int32_t H, int32_t k, int32_t block,
                            int32_t n_blocks, int32_t* topk, int32_t* pool, int32_t* pool_len, float* scores_opt,
                            void* ws, size_t ws_bytes, void* stream) {
  if (Q < 1 || Q > CSA2_MAX_QUERIES_PER_SEQ) return CSA2_ERR_SHAPE;
  if (B < 0 || (int64_t)B * Q > INT32_MAX || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !q_codes || !q_scales || !w || !topk) return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_len)) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q_codes)) return CSA2_ERR_ALIGN;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_mq_workspace(B, Q, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full(idx_codes, idx_scales, cap, len, B * Q, nullptr, q_codes, q_scales, w,
                                          H, k, block, n_blocks, topk, pool, pool_len, scores_opt, ws,
                                          as_stream(stream), Q));
}

int csa2_index_full_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                         const int32_t* len, int32_t B, const uint8_t* q_codes,
                         const uint8_t* q_scales, const float* w, int32_t H, int32_t k,
                         int32_t block, int32_t n_blocks, int32_t* topk, int32_t* pool,
                         int32_t* pool_len, float* scores_opt, void* ws, size_t ws_bytes,
                         void* stream) {
  if (B < 0 || cap < 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !q_codes || !q_scales || !w || !topk) return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_len)) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q_codes)) return CSA2_ERR_ALIGN;
  if (cap == 0) return CSA2_ERR_SHAPE;
  if (!ws || ws_bytes < csa2_index_full_workspace(B, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full(idx_codes, idx_scales, cap, len, B, nullptr, q_codes, q_scales, w,
                                          H, k, block, n_blocks, topk, pool, pool_len, scores_opt, ws,
                                          as_stream(stream)));
}

size_t csa2_index_pool_workspace(int32_t B, int32_t pool_cap, int32_t k) {
  (void)k;
  if (B <= 0 || pool_cap <= 0) return 0;
  return csa2::index_pool_ws_bytes(B, pool_cap);
}

int csa2_index_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                    const int32_t* len, int32_t B, const int32_t* pool, const int32_t* pool_len,
                    int32_t pool_cap, const uint16_t* q, const float* w, int32_t H, int32_t k,
                    int32_t* topk, float* pool_scores_opt, void* ws, size_t ws_bytes,
                    void* stream) {
  if (B < 0 || cap <= 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !pool || !pool_len || !q || !w || !topk)
    return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  const size_t need = csa2_index_pool_workspace(B, pool_cap, k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool(idx_codes, idx_scales, cap, len, B, pool, pool_len,
                                          pool_cap, q, nullptr, nullptr, w, H, k, topk, pool_scores_opt,
                                          ws, as_stream(stream)));
}

static int index_pool_mq(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                         int32_t B, int32_t Q, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                         bool fp4q, const uint16_t* q, const uint8_t* q_codes, const uint8_t* q_scales,
                         const float* w, int32_t H, int32_t k, int32_t* topk, float* pool_scores_opt, void* ws,
                         size_t ws_bytes, void* stream) {
  if (Q < 1 || Q > CSA2_MAX_QUERIES_PER_SEQ) return CSA2_ERR_SHAPE;
  if (B < 0 || (int64_t)B * Q > INT32_MAX || cap <= 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !pool || !pool_len || !w || !topk) return CSA2_ERR_NULL;
  if (fp4q ? (!q_codes || !q_scales) : !q) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(fp4q ? (const void*)q_codes : (const void*)q))
    return CSA2_ERR_ALIGN;
  const size_t need = csa2_index_pool_workspace(B * Q, pool_cap, k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool(idx_codes, idx_scales, cap, len, B * Q, pool, pool_len, pool_cap,
                                          fp4q ? nullptr : q, fp4q ? q_codes : nullptr, fp4q ? q_scales : nullptr,
                                          w, H, k, topk,
                                          pool_scores_opt, ws, as_stream(stream), nullptr, nullptr, Q));
}

int csa2_index_pool_mq(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                       int32_t B, int32_t Q, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                       const uint16_t* q, const float* w, int32_t H, int32_t k, int32_t* topk,
                       float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream) {
  return index_pool_mq(idx_codes, idx_scales, cap, len, B, Q, pool, pool_len, pool_cap, false, q, nullptr, nullptr,
                       w, H, k, topk, pool_scores_opt, ws, ws_bytes, stream);
}

int csa2_index_pool_mq_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                            int32_t B, int32_t Q, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                            const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int32_t H, int32_t k,
                            int32_t* topk, float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream) {
  return index_pool_mq(idx_codes, idx_scales, cap, len, B, Q, pool, pool_len, pool_cap, true, nullptr, q_codes,
                       q_scales, w, H, k, topk, pool_scores_opt, ws, ws_bytes, stream);
}

int csa2_index_pool_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                          int32_t B, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                          const uint16_t* q, const float* w, int32_t H, float* pool_scores_opt, void* ws,
                          size_t ws_bytes, void* stream) {
  if (B < 0 || cap <= 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !pool || !pool_len || !q || !w) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  const size_t need = csa2_index_pool_workspace(B, pool_cap, 1);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool_score(idx_codes, idx_scales, cap, len, B, pool, pool_len, pool_cap, q,
                                                nullptr, nullptr, w, H, pool_scores_opt, ws, as_stream(stream)));
}

int csa2_index_pool_select(int32_t B, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap, int32_t k,
                           int32_t* topk, const float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!pool || !pool_len || !topk) return CSA2_ERR_NULL;
  const size_t need = csa2_index_pool_workspace(B, pool_cap, k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool_select(B, pool, pool_len, pool_cap, k, topk, pool_scores_opt, ws,
                                                 as_stream(stream)));
}

int csa2_index_pool_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                         const int32_t* len, int32_t B, const int32_t* pool, const int32_t* pool_len,
                         int32_t pool_cap, const uint8_t* q_codes, const uint8_t* q_scales,
                         const float* w, int32_t H, int32_t k, int32_t* topk, float* pool_scores_opt,
                         void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || cap <= 0 || cap > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !len || !pool || !pool_len || !q_codes || !q_scales || !w || !topk)
    return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q_codes)) return CSA2_ERR_ALIGN;
  const size_t need = csa2_index_pool_workspace(B, pool_cap, k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool(idx_codes, idx_scales, cap, len, B, pool, pool_len,
                                          pool_cap, nullptr, q_codes, q_scales, w, H, k, topk,
                                          pool_scores_opt, ws, as_stream(stream)));
}

size_t csa2_attn_workspace(int32_t B, int32_t H, int32_t k, int32_t swa_cap) {
  if (B <= 0 || H <= 0 || k < 0 || swa_cap < 0) return 0;
  return csa2::attn_ws_bytes(B, H, k, swa_cap);
}

int csa2_sparse_attn_decode(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                            const uint8_t* main_scales, int64_t cap, int32_t main_fmt,
                            const int32_t* len, const int32_t* topk, int32_t k, int32_t B,
                            const uint8_t* swa_codes, const uint8_t* swa_scales,
                            int64_t swa_stride, int32_t swa_cap, const int32_t* swa_len,
                            int32_t swa_fmt, float sm_scale, const int64_t* q_pos, uint16_t* out,
                            float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn(q, H, main_codes, main_scales, cap, CSA2_MAX_CACHE_ROWS, main_fmt, true, len, topk, k,
                            B, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale, q_pos, out);
  if (rc != CSA2_OK || B == 0) return rc;
  if (!ws || ws_bytes < csa2_attn_workspace(B, H, k, swa_cap)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_sparse_attn(q, H, main_codes, main_scales, cap, main_fmt, len, topk,
                                           k, B, swa_codes, swa_scales, swa_stride, swa_cap,
                                           swa_len, swa_fmt, sm_scale, q_pos, out, lse_opt, ws,
                                           as_stream(stream)));
}

int csa2_sparse_attn_decode_mq(const uint16_t* q, int32_t H, int32_t Q, const uint8_t* main_codes,
                               const uint8_t* main_scales, int64_t cap, int32_t main_fmt, const int32_t* len,
                               const int32_t* topk, int32_t k, int32_t B, const uint8_t* swa_codes,
                               const uint8_t* swa_scales, int64_t swa_stride, int32_t swa_cap,
                               const int32_t* swa_len, int32_t swa_fmt, float sm_scale, const int64_t* q_pos,
                               uint16_t* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  if (Q < 1 || Q > CSA2_MAX_QUERIES_PER_SEQ || B < 0 || (int64_t)B * Q > INT32_MAX) return CSA2_ERR_SHAPE;
  const int32_t R = B * Q;  // query rows
  const int rc = check_attn(q, H, main_codes, main_scales, cap, CSA2_MAX_CACHE_ROWS, main_fmt, true, len, topk, k,
                            R, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale, q_pos, out);
  if (rc != CSA2_OK || B == 0) return rc;
  if (!ws || ws_bytes < csa2_attn_workspace(R, H, k, swa_cap)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_sparse_attn(q, H, main_codes, main_scales, cap, main_fmt, len, topk, k, R,
                                           swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale,
                                           q_pos, out, lse_opt, ws, as_stream(stream), false, Q));
}

int csa2_sparse_attn_decode_noalloc(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                                    const uint8_t* main_scales, int64_t cap, int32_t main_fmt,
                                    const int32_t* len, const int32_t* topk, int32_t k, int32_t B,
                                    const uint8_t* swa_codes, const uint8_t* swa_scales,
                                    int64_t swa_stride, int32_t swa_cap, const int32_t* swa_len,
                                    int32_t swa_fmt, float sm_scale, const int64_t* q_pos, uint16_t* out,
                                    float* lse_opt, void* stream) {
  const int rc = check_attn(q, H, main_codes, main_scales, cap, CSA2_MAX_CACHE_ROWS, main_fmt, true, len, topk, k,
                            B, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale, q_pos, out);
  if (rc != CSA2_OK || B == 0) return rc;
  if (csa2_attn_workspace(B, H, k, swa_cap) > (size_t)CSA2_ATTN_NOALLOC_SCRATCH_BYTES) return CSA2_ERR_SCRATCH;
  int src = CSA2_OK;
  void* ws = device_scratch(as_stream(stream), &src);
  if (!ws) return src;
  return launched(csa2::launch_sparse_attn(q, H, main_codes, main_scales, cap, main_fmt, len, topk,
                                           k, B, swa_codes, swa_scales, swa_stride, swa_cap,
                                           swa_len, swa_fmt, sm_scale, q_pos, out, lse_opt, ws,
                                           as_stream(stream)));
}

// ------------------------------------------------------------ paged cache
// A valid page map: pages of 2^page_shift entries (64 .. 2^20), a logical
// capacity of at most CSA2_MAX_CACHE_ROWS entries, and a pool of whole pages
// small enough for 32-bit byte offsets into the 64-byte indexer-K rows.
static int paged_shape(int64_t n_rows, int32_t page_shift, int32_t max_pages) {
  if (page_shift < CSA2_MIN_PAGE_SHIFT || page_shift > CSA2_MAX_PAGE_SHIFT || max_pages < 1) return CSA2_ERR_SHAPE;
  if (((int64_t)max_pages << page_shift) > CSA2_MAX_CACHE_ROWS) return CSA2_ERR_SHAPE;
  if (n_rows < (1 << page_shift) || n_rows > CSA2_MAX_POOL_ROWS || (n_rows & ((1 << page_shift) - 1)))
    return CSA2_ERR_SHAPE;
  return CSA2_OK;
}

static csa2::PageMap page_map(const int32_t* table, int64_t n_rows, int32_t page_shift, int32_t max_pages) {
  return csa2::PageMap{table, page_shift, max_pages, (int32_t)(n_rows >> page_shift)};
}

int csa2_cache_append_paged(const uint16_t* latent, const uint16_t* gate, int32_t B, int32_t m,
                            const float* gamma, float eps, const float* w_idx, int32_t main_fmt, int32_t rope,
                            uint8_t* main_codes, uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales,
                            int64_t n_rows, const int32_t* block_table, int32_t page_shift, int32_t max_pages,
                            int32_t* len, void* state, void* stream) {
  const int ps = paged_shape(n_rows, page_shift, max_pages);
  if (ps != CSA2_OK) return ps;
  if (B < 0 || m < 1 || m > 2) return CSA2_ERR_SHAPE;
  if (!valid_fmt(main_fmt)) return CSA2_ERR_UNSUPPORTED;
  if (!(eps >= 0.0f)) return CSA2_ERR_SHAPE;
  if (B == 0) return CSA2_OK;
  if (!latent || (m == 2 && (!gate || !state)) || !w_idx || !main_codes || !main_scales || !idx_codes ||
      !idx_scales || !len || !block_table)
    return CSA2_ERR_NULL;
  if (!aligned16(latent) || (m == 2 && (!aligned16(gate) || !aligned16(state))) || !aligned16(main_codes) ||
      !aligned16(idx_codes) || (reinterpret_cast<uintptr_t>(w_idx) & 3u) ||
      (reinterpret_cast<uintptr_t>(len) & 3u) || (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return CSA2_ERR_ALIGN;
  const int64_t cap = (int64_t)max_pages << page_shift;
  return launched(csa2::launch_cache_append(latent, gate, B, m, gamma, eps, w_idx, main_fmt, rope ? 1 : 0,
                                            main_codes, main_scales, idx_codes, idx_scales, cap, len, state,
                                            as_stream(stream), page_map(block_table, n_rows, page_shift, max_pages)));
}

int csa2_index_full_paged(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t n_rows,
                          const int32_t* block_table, int32_t page_shift, int32_t max_pages,
                          const int32_t* len, int32_t B, const uint16_t* q, const float* w, int32_t H,
                          int32_t k, int32_t block, int32_t n_blocks, int32_t* topk, int32_t* topk_rows,
                          int32_t* pool, int32_t* pool_rows, int32_t* pool_len, float* scores_opt,
                          void* ws, size_t ws_bytes, void* stream) {
  const int ps = paged_shape(n_rows, page_shift, max_pages);
  if (ps != CSA2_OK) return ps;
  const int64_t cap = (int64_t)max_pages << page_shift;
  if (B < 0) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
  if (n_blocks < 0 || n_blocks > CSA2_POOL_BLOCKS || (int64_t)n_blocks * block > CSA2_MAX_POOL)
    return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !block_table || !len || !q || !w || !topk || !topk_rows)
    return CSA2_ERR_NULL;
  if (n_blocks > 0 && (!pool || !pool_rows || !pool_len)) return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q) ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return CSA2_ERR_ALIGN;
  if (!ws || ws_bytes < csa2_index_full_workspace(B, cap, k, block, n_blocks)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_full(idx_codes, idx_scales, cap, len, B, q, nullptr, nullptr, w, H, k, block,
                                          n_blocks, topk, pool, pool_len, scores_opt, ws, as_stream(stream), 1,
                                          page_map(block_table, n_rows, page_shift, max_pages), topk_rows,
                                          n_blocks > 0 ? pool_rows : nullptr));
}

int csa2_index_pool_rows(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t n_rows, int32_t B,
                         const int32_t* pool, const int32_t* pool_rows, const int32_t* pool_len,
                         int32_t pool_cap, const uint16_t* q, const float* w, int32_t H, int32_t k,
                         int32_t* topk, int32_t* topk_rows, float* pool_scores_opt, void* ws, size_t ws_bytes,
                         void* stream) {
  if (B < 0 || n_rows <= 0 || n_rows > CSA2_MAX_POOL_ROWS) return CSA2_ERR_SHAPE;
  if (pool_cap < 0 || pool_cap > CSA2_MAX_POOL) return CSA2_ERR_SHAPE;
  if (k < 1 || k > CSA2_MAX_TOPK) return CSA2_ERR_SHAPE;
  if (!valid_index_heads(H)) return CSA2_ERR_UNSUPPORTED;
  if (B == 0) return CSA2_OK;
  if (!idx_codes || !idx_scales || !pool || !pool_rows || !pool_len || !q || !w || !topk || !topk_rows)
    return CSA2_ERR_NULL;
  if (!aligned16(idx_codes) || !aligned16(idx_scales) || !aligned16(q)) return CSA2_ERR_ALIGN;
  const size_t need = csa2_index_pool_workspace(B, pool_cap, k);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_index_pool(idx_codes, idx_scales, n_rows, nullptr, B, pool, pool_len, pool_cap, q,
                                          nullptr, nullptr, w, H, k, topk, pool_scores_opt, ws, as_stream(stream),
                                          pool_rows, topk_rows));
}

int csa2_sparse_attn_decode_rows(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                                 const uint8_t* main_scales, int64_t n_rows, int32_t main_fmt,
                                 const int32_t* rows, int32_t k, int32_t B, const uint8_t* swa_codes,
                                 const uint8_t* swa_scales, int64_t swa_stride, int32_t swa_cap,
                                 const int32_t* swa_len, int32_t swa_fmt, float sm_scale, const int64_t* q_pos,
                                 uint16_t* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream) {
  const int rc = check_attn(q, H, main_codes, main_scales, n_rows, CSA2_MAX_POOL_ROWS, main_fmt, false, nullptr,
                            rows, k, B, swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale,
                            q_pos, out);
  if (rc != CSA2_OK || B == 0) return rc;
  if (!ws || ws_bytes < csa2_attn_workspace(B, H, k, swa_cap)) return CSA2_ERR_WORKSPACE;
  return launched(csa2::launch_sparse_attn(q, H, main_codes, main_scales, n_rows, main_fmt, nullptr, rows, k, B,
                                           swa_codes, swa_scales, swa_stride, swa_cap, swa_len, swa_fmt, sm_scale,
                                           q_pos, out, lse_opt, ws, as_stream(stream), true));
}

}  // extern "C"
