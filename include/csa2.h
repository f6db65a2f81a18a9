/*
 * csa2.h -- C ABI of the CSA2 decode hot path over an FP4 global KV cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages on DeepSeek V4.1 Flash; cited by host, title and section):
 *   [JU]  jokeuncle.pages.dev, "两张架构图里藏着 890 字节", sections 二, 三, 四
 *   [WG]  weigao.cc, "DeepSeek V4.1 Flash：从架构到推理成本", sections 3.1, 3.2, 4, 7, 10
 *   [SY]  syt-nju.github.io, "DeepSeek-V4.1-Flash：为什么读输入只激活 8B，写输出要 16B",
 *         sections "CSA2" (Figure 4), "Hierarchical Sparse Indexer" (Figure 5),
 *         "FP4 主 KV 缓存" (Figure 1(b))
 *   [GP]  ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析", sections 3.2, 3.3, 4.1, 7
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA tensor).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work on `stream`; none of them synchronises.
 *  - The caller owns every buffer, including the workspace; the library holds
 *    no state and allocates nothing, so calls are re-entrant.  Two calls that
 *    share a workspace must be ordered on one stream.
 *  - Return value: CSA2_OK or an error code.  Host-side validation runs before
 *    any launch; on a validation error nothing is launched and no output is
 *    written.  CSA2_ERR_HIP reports a launch failure; faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - Device-side lengths (`len`, `swa_len`, `pool_len`) are clamped to their
 *    buffer capacities; device-side indices outside [0, len_b) or equal to -1
 *    are masked (never dereferenced, never selected, never attended).
 *
 * FP4 cache planes (structure-of-arrays, one plane per field)
 * ----------------------------------------------------------
 *  An FP4 row of `dim` values is stored as
 *     codes  : dim/2 bytes; value 2i in bits 0-3, value 2i+1 in bits 4-7;
 *              each nibble is E2M1 (sign, 2 exponent bits, 1 mantissa bit,
 *              magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6})          [JU 三 事实一]
 *     scales : dim/group bytes, one per consecutive `group` values.
 *  value = e2m1(code) * scale(byte).
 *  Main KV    : dim 512, group 16 -> 256 + 32 = 288 B per entry; the scale byte is
 *               E4M3 on the pages [JU 三 事实一; SY FP4 主 KV 缓存; GP 7] or E8M0
 *               ("MXFP4") -- both are supported, chosen by `main_fmt`.
 *  Indexer K  : dim 128, group 32, E8M0 -> 64 + 4 = 68 B per entry [JU 三 事实二].
 *  A cache for B sequences of capacity `cap` entries is laid out
 *     main_codes [B][cap][256], main_scales [B][cap][32],
 *     idx_codes  [B][cap][64],  idx_scales  [B][cap][4].
 *  Planes must be 16-byte aligned.
 *
 * Quantisation rule (the pages fix the format, not the rounding; readings):
 *  scale = the smallest representable scale s with 6*s >= max|x| over the
 *  group (E8M0: s = 2^(b-127), b in [0,254]; E4M3: OCP E4M3FN finite codes
 *  0x00..0x7E); the maximum code when none qualifies; code 0 when max|x| = 0.
 *  Each |x|/s is rounded to the nearest E2M1 magnitude, ties to the even code;
 *  a zero magnitude always encodes as +0 (code 0).
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- constants of the published configuration [JU 二 config map; JU 三] ---- */
#define CSA2_MAIN_DIM 512          /* head_dim of the compressed main KV          */
#define CSA2_MAIN_GROUP 16         /* values per main-KV scale byte               */
#define CSA2_MAIN_CODE_BYTES 256   /* 512 values x 4 bit                          */
#define CSA2_MAIN_SCALE_BYTES 32   /* 512 / 16                                    */
#define CSA2_IDX_DIM 128           /* index_head_dim                              */
#define CSA2_IDX_GROUP 32          /* values per indexer-K scale byte (E8M0)      */
#define CSA2_IDX_CODE_BYTES 64
#define CSA2_IDX_SCALE_BYTES 4
#define CSA2_INDEX_TOPK 512        /* index_topk                                  */
#define CSA2_BLOCK 8               /* candidate_block_size                        */
#define CSA2_POOL_BLOCKS 2048      /* candidate_topk_blocks                       */
#define CSA2_SWA 128               /* sliding_window                              */
#define CSA2_WIN_DATA_BYTES 576    /* FP8 window record: 448 E4M3 + 64 x bf16     */
#define CSA2_WIN_SCALE_BYTES 8     /* 7 UE8M0 scales (one per 64 dims) + 1 pad    */
#define CSA2_SWA_MAIN 0            /* window rows in the main-KV format           */
#define CSA2_SWA_FP8 1             /* window rows as FP8 records                  */
#define CSA2_ATTN_HEADS 64         /* query heads of the core attention           */

#define CSA2_MAX_TOPK 2048
#define CSA2_MAX_POOL 16384        /* n_blocks * block upper bound                */
#define CSA2_MAX_QUERIES_PER_SEQ 16 /* queries sharing one cache (the *_mq calls) */
#define CSA2_MIN_PAGE_SHIFT 6      /* paged cache: pages of 2^6 .. 2^20 entries    */
#define CSA2_MAX_PAGE_SHIFT 20
#define CSA2_MAX_POOL_ROWS (1 << 26) /* rows of a paged pool (32-bit byte offsets)  */
#define CSA2_MAX_CACHE_ROWS 1048576 /* entries per sequence accepted by index_full */
#define CSA2_ATTN_MAX_GROUPS 65536  /* B * H / 16 accepted by csa2_sparse_attn_decode  */
#define CSA2_ATTN_WS_COUNTER_BYTES (CSA2_ATTN_MAX_GROUPS * 4) /* leading zeroed region */
#define CSA2_ATTN_NOALLOC_SCRATCH_BYTES (32 << 20) /* per-GPU scratch of csa2_sparse_attn_decode_noalloc */

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,        /* a required pointer is NULL                        */
  CSA2_ERR_SHAPE = 2,       /* a size argument is out of range or inconsistent   */
  CSA2_ERR_ALIGN = 3,       /* a plane pointer is not 16-byte aligned            */
  CSA2_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. head count)       */
  CSA2_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  CSA2_ERR_HIP = 6,         /* a HIP launch failed                               */
  CSA2_ERR_SCRATCH = 7      /* larger than the library's fixed scratch (noalloc) */
} csa2_status;

typedef enum { CSA2_SCALE_E8M0 = 0, CSA2_SCALE_E4M3 = 1 } csa2_scale_fmt;

/* Human-readable name of a status code (static string; never NULL). */
const char* csa2_status_string(int status);

/* Library version, as "csa2 <major>.<minor> gfx950". */
const char* csa2_version(void);

/*
 * csa2_quantize_fp4 -- FP4 (E2M1) quantisation of fp32 rows with one scale
 * byte per `group` values.  It is the quantiser the cache write applies to the
 * main KV and to the indexer K [JU 三 事实一, 事实二; GP 7].
 *   x      : fp32 [rows][dim], row-major.
 *   dim    : multiple of `group`; group is 16 or 32; dim <= 4096.
 *   fmt    : CSA2_SCALE_E8M0 or CSA2_SCALE_E4M3.
 *   codes  : out, u8 [rows][dim/2].   scales : out, u8 [rows][dim/group].
 * Errors: NULL pointer, rows < 0, bad dim/group/fmt, misaligned x/codes.
 */
int csa2_quantize_fp4(const float* x, int64_t rows, int32_t dim, int32_t group,
                      int32_t fmt, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * csa2_cache_write -- the compressor of a KV-source (Full) layer writing T
 * tokens as T/m compressed entries [JU 四 item 1; GP 3.2 (Z); SY CSA2]:
 *   for group j (tokens m*j .. m*j+m-1) and channel c:
 *     pooled[c] = sum_t softmax_t(gate[t][c]) * latent[t][c]   (fp32; m == 1: latent)
 *     y = pooled * rsqrt(mean_c(pooled^2) + eps) * gamma        (RMSNorm)
 *     main entry = FP4(y), group 16, scale format `main_fmt`
 *     k = y @ w_idx (512 -> 128, fp32)  -> FP4(k), group 32, E8M0 (indexer K)
 *   latent, gate : bf16 bits [T][512]; gate is not read when m == 1 (may be NULL).
 *   m            : tokens per entry, 1..8; T must be a multiple of m.
 *   gamma        : fp32 [512] RMSNorm weight, NULL = all ones.
 *   w_idx        : fp32 [512][128] indexer-K projection (row c, column d),
 *                  16-byte aligned.
 *   rope_pos     : int64 [T/m] position of each written entry, or NULL.  With
 *                  positions, the main entry's dims 448..511 are rotated by the
 *                  compressed RoPE before FP4 [GP 3.2 (RMSNorm -> RoPE base
 *                  160000 -> FP4), GP 7 (448 dims without position, 64 with)]:
 *                  32 adjacent pairs (448+2j, 449+2j) turned by
 *                  pos * 160000^(-2j/64).  The indexer key is projected from the
 *                  entry before rotation.  8-byte aligned.
 *   main_codes/main_scales/idx_codes/idx_scales : out, rows [T/m] of the
 *                  planes above, i.e. pointers to the destination entry.
 * Errors: NULL pointer, T < 0, T % m != 0, m outside 1..8, bad main_fmt,
 *         misaligned planes.
 */
int csa2_cache_write(const uint16_t* latent, const uint16_t* gate, int64_t T, int32_t m,
                     const float* gamma, float eps, const float* w_idx, int32_t main_fmt,
                     const int64_t* rope_pos, uint8_t* main_codes, uint8_t* main_scales,
                     uint8_t* idx_codes, uint8_t* idx_scales, void* stream);

/*
 * csa2_cache_append -- decode-time append [JU 四 item 1; GP 3.2]: one new
 * token per sequence.  A decoder layer (m = 1) writes one compressed entry
 * per token; a layer with m = 2 writes one entry per two tokens and holds
 * the first token of each group in `state` until its partner arrives.
 *   latent, gate : bf16 bits [B][512], the new token of each sequence (gate
 *                  is read only when m == 2).
 *   m            : 1 or 2.
 *   gamma, eps, w_idx, main_fmt : as csa2_cache_write.
 *   rope         : non-zero to rotate each written entry by the compressed
 *                  RoPE at its own row index len[b] (csa2_cache_write's
 *                  rope_pos, with the entry index as the position).
 *   main_codes/main_scales/idx_codes/idx_scales : the cache planes
 *                  [B][cap][256] / [B][cap][32] / [B][cap][64] / [B][cap][4].
 *   len          : int32 [B], in/out.  A written entry goes to row len[b] and
 *                  len[b] then grows by one.  A sequence with len[b] >= cap is
 *                  full: nothing is written or held, and len[b] stays.
 *   state        : m == 2 only (else may be NULL): csa2_append_state_bytes(B)
 *                  bytes, zero-filled once before the first call, then owned
 *                  by the calls (per sequence: tokens held, and the held
 *                  token's latent and gate).  16-byte aligned.
 * The entry written equals csa2_cache_write of the group's tokens.  Two
 * launches on `stream` (the write, then the advance of len/state); no
 * allocation, no memset, so it may be captured in a graph.  Calls sharing
 * `len` or `state` must be ordered on one stream.
 */
size_t csa2_append_state_bytes(int32_t B);
int csa2_cache_append(const uint16_t* latent, const uint16_t* gate, int32_t B, int32_t m,
                      const float* gamma, float eps, const float* w_idx, int32_t main_fmt, int32_t rope,
                      uint8_t* main_codes, uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales,
                      int64_t cap, int32_t* len, void* state, void* stream);

/*
 * csa2_window_write -- the FP8 sliding-window ring of one layer [GP 4.1: a
 * 128-token window whose entries stay in FP8; GP 7: 448 B position-free + 128 B
 * RoPE + 8 B scale = 584 B per token, 576-B aligned; WG 10.1: the FP8 window
 * record stays beside an FP4 compressed cache; JU 顺便算清另外三笔账: 128 slots
 * per sequence, overwritten as a ring].  Writes n new tokens per sequence.
 *   latent   : bf16 bits [B][n][512], token i of sequence b at position
 *              pos0[b] + i.  16-byte aligned.
 *   gamma, eps : RMSNorm weight (fp32 [512], NULL = 1) and epsilon (>= 0): the
 *              window row is the token's RMS-normalised latent (the m = 1
 *              arithmetic of csa2_cache_write: no pooling).
 *   rope     : non-zero to rotate dims 448..511 by the compressed RoPE at the
 *              token's position before storing.
 *   pos0     : int64 [B], position of token 0 of each sequence (8-byte aligned).
 *              A sequence with pos0[b] < 0 is left untouched.
 *   W        : slots per sequence, 1..128; token at position p goes to slot
 *              p mod W, so the ring holds the last min(p + 1, W) tokens.
 *   win_data : u8 [B][W][576] records: bytes 0..447 are OCP E4M3 codes of dims
 *              0..447 (nearest, ties to even, a zero magnitude as +0), bytes
 *              448..575 dims 448..511 as bf16 (nearest even).  16-byte aligned.
 *   win_scales : u8 [B][W][8]: byte i (i < 7) is the UE8M0 scale 2^(s-127) of
 *              dims 64i..64i+63, the smallest with 448 * scale >= the group's
 *              largest magnitude (0 for an all-zero group); byte 7 is 0.
 *              8-byte aligned.
 *   swa_len  : out int32 [B]: min(pos0[b] + n, W), the rows the window holds.
 * Only the last min(n, W) tokens are written (an earlier one would be
 * overwritten in the same call).  One launch on `stream`; no allocation.
 * Errors: B < 0, n < 0, W outside 1..128, eps < 0, NULL or misaligned planes.
 */
int csa2_window_write(const uint16_t* latent, int32_t B, int32_t n, const float* gamma, float eps,
                      int32_t rope, const int64_t* pos0, int32_t W, uint8_t* win_data,
                      uint8_t* win_scales, int32_t* swa_len, void* stream);

/*
 * csa2_index_full -- Full-mode hierarchical sparse indexer: one scoring pass
 * over every visible entry, feeding two selections [GP 3.3; SY Figure 5; WG 3.2]:
 *   score[b][p] = sum_h w[b][h] * max(0, q[b][h] . deq(idx K[b][p]))  for p < len[b]
 *   topk[b]  : the k positions of highest score (ties: lower position first),
 *              written in ascending position order, -1 padded when len[b] < k.
 *   blocks   : block i covers positions [block*i, block*i+block) ∩ [0, len[b]);
 *              its score is the maximum member score (an upper bound of each).
 *              The n_blocks highest-scoring blocks (ties: lower block first) are
 *              expanded into pool[b] (ascending positions, -1 padded to
 *              n_blocks*block); pool_len[b] = number of positions written.
 *   idx_codes/idx_scales : indexer-K planes [B][cap][64] / [B][cap][4].
 *   len      : int32 [B] visible entries per sequence (device).
 *   q        : bf16 bits [B][H][128] indexer queries; w : fp32 [B][H] head weights.
 *   H        : 8, 16, 32 or 64.   k : 1..2048.   block : 8.
 *   n_blocks : 0..2048 with n_blocks*block <= 16384; 0 = no pool.
 *   topk     : out int32 [B][k].
 *   pool, pool_len : out int32 [B][n_blocks*block], [B] (may be NULL iff n_blocks == 0).
 *   scores_opt : optional out fp32 [B][cap]; entries p >= len[b] are unspecified.
 *   ws, ws_bytes : workspace of at least csa2_index_full_workspace(...) bytes.
 */
size_t csa2_index_full_workspace(int32_t B, int64_t cap, int32_t k, int32_t block,
                                 int32_t n_blocks);
int csa2_index_full(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                    const int32_t* len, int32_t B, const uint16_t* q, const float* w,
                    int32_t H, int32_t k, int32_t block, int32_t n_blocks, int32_t* topk,
                    int32_t* pool, int32_t* pool_len, float* scores_opt, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * csa2_index_full_score / csa2_index_full_select -- the two phases of
 * csa2_index_full as separate calls, for callers that want the scores alone,
 * or that select from scores scored elsewhere (e.g. each GPU scoring its own
 * share of a long sequence), or that time the phases apart.  The pages' "one
 * scoring pass feeds both selections" [GP 3.3] is the pair called in order
 * on one workspace; together they launch exactly the kernels of
 * csa2_index_full and give bit-identical results.
 *   csa2_index_full_score: arguments as csa2_index_full (no k, n_blocks or
 *     outputs); writes every visible entry's score (to scores_opt when given,
 *     else into ws) and the maximum of every 8-entry block (into ws).
 *   csa2_index_full_select: the position top-k and the block pool of
 *     csa2_index_full from those; scores_opt must be the pointer the scoring
 *     call was given (or NULL if it had none), ws the same workspace
 *     (csa2_index_full_workspace bytes) holding the block maxima.
 */
int csa2_index_full_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                          int32_t B, const uint16_t* q, const float* w, int32_t H, int32_t block, float* scores_opt,
                          void* ws, size_t ws_bytes, void* stream);
int csa2_index_full_select(int64_t cap, const int32_t* len, int32_t B, int32_t k, int32_t block, int32_t n_blocks,
                           int32_t* topk, int32_t* pool, int32_t* pool_len, const float* scores_opt, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * csa2_index_pool -- Reindex mode: a layer's own indexer query rescored over
 * the shared candidate pool only, then its own top-k [SY Figure 5 (right);
 * GP 3.3; SY CSA2 Figure 4 (Reindex)].  Same score formula as index_full.
 *   pool     : int32 [B][pool_cap] positions (from csa2_index_full); entries
 *              i < pool_len[b] are candidates; -1 or out-of-range are masked.
 *              Precondition: the valid entries of a row appear in strictly
 *              ascending order (csa2_index_full writes them so); masked entries
 *              may appear anywhere.  Ties and output order rely on it.
 *   topk     : out int32 [B][k] ascending positions, -1 padded; ties prefer
 *              the lower position.
 *   pool_scores_opt : optional out fp32 [B][pool_cap] (score of pool[b][i]).
 *   H, k as for csa2_index_full; pool_cap <= 16384.
 *   ws, ws_bytes : workspace of at least csa2_index_pool_workspace(...) bytes
 *              (pool scores unless pool_scores_opt is given, and the maxima
 *              of groups of 8 consecutive pool entries); required in every
 *              call with pool_cap > 0; no initial contents needed.
 * Selection goes through the top-k groups of 8 consecutive pool entries
 * (group score = max); the position top-k is exact over their entries.
 */
size_t csa2_index_pool_workspace(int32_t B, int32_t pool_cap, int32_t k);
int csa2_index_pool(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                    const int32_t* len, int32_t B, const int32_t* pool,
                    const int32_t* pool_len, int32_t pool_cap, const uint16_t* q,
                    const float* w, int32_t H, int32_t k, int32_t* topk,
                    float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_pool_mq -- csa2_index_pool for Q queries per sequence (the draft
 * positions of a verify block [WG 7]), each rescoring its own pool (as
 * csa2_index_full_mq returns them) over its sequence's cache, in one call.
 *   pool     : int32 [B][Q][pool_cap];  pool_len : int32 [B][Q];
 *   q        : bf16 bits [B][Q][H][128];  w : fp32 [B][Q][H];
 *   topk     : out int32 [B][Q][k];  pool_scores_opt : out fp32 [B][Q][pool_cap].
 *   idx planes and len [B] are per sequence.  Q : 1..CSA2_MAX_QUERIES_PER_SEQ.
 *   ws       : at least csa2_index_pool_workspace(B*Q, pool_cap, k) bytes.
 * Query row (b, i) gives exactly what csa2_index_pool gives for row i of the
 * sequence alone; with Q = 1 this is csa2_index_pool.  The scoring kernel
 * places a sequence's Q rows side by side (as in csa2_index_full_mq).
 * Errors: as csa2_index_pool; Q outside 1..CSA2_MAX_QUERIES_PER_SEQ is
 * CSA2_ERR_SHAPE.
 */
int csa2_index_pool_mq(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                       int32_t B, int32_t Q, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                       const uint16_t* q, const float* w, int32_t H, int32_t k, int32_t* topk,
                       float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream);
/*
 * csa2_index_pool_mq_fp4q -- csa2_index_pool_mq with FP4 indexer queries, as
 * csa2_index_pool_fp4q takes them [syt-nju.github.io, section FP4 主 KV 缓存]:
 *   q_codes  : u8 [B][Q][H][64] E2M1 codes, 16-byte aligned;
 *   q_scales : u8 [B][Q][H][4] E8M0 scale bytes, one per 32 dims.
 * Every other argument, the outputs and the status codes are those of
 * csa2_index_pool_mq; query row (b, i) equals csa2_index_pool_fp4q on row i
 * of the sequence alone.
 */
int csa2_index_pool_mq_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                            int32_t B, int32_t Q, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                            const uint8_t* q_codes, const uint8_t* q_scales, const float* w, int32_t H, int32_t k,
                            int32_t* topk, float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_pool_score / csa2_index_pool_select -- the two phases of
 * csa2_index_pool as separate calls (as for csa2_index_full_score/_select):
 * the pool rescoring (pool scores to pool_scores_opt when given, else into
 * ws, and the maxima of groups of 8 consecutive pool entries into ws), then
 * the layer's top-k from them.  The select call takes the same pool,
 * pool_len, pool_scores_opt and workspace.
 */
int csa2_index_pool_score(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap, const int32_t* len,
                          int32_t B, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap,
                          const uint16_t* q, const float* w, int32_t H, float* pool_scores_opt, void* ws,
                          size_t ws_bytes, void* stream);
int csa2_index_pool_select(int32_t B, const int32_t* pool, const int32_t* pool_len, int32_t pool_cap, int32_t k,
                           int32_t* topk, const float* pool_scores_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_full_mq -- the Full-mode indexer for Q queries of each sequence
 * at once, such as the positions of a speculative verify block [WG 7: the
 * draft block has 5 parallel positions (dspark_block_size); JU 四 item 2: the
 * 5-position block runs in one forward].  Query i of sequence b gets exactly
 * what csa2_index_full gives it against cache b:
 *   score[b][i][p] = sum_h w[b][i][h] * max(0, q[b][i][h] . deq(idx K[b][p]))  for p < len[b]
 * with its own top-k and pool under the same rules.  The Q queries of a
 * sequence walk the cache's entries side by side, so the cache is read from
 * HBM about once for all of them (the others find it in L2).
 *   B        : sequences (caches);  Q : queries per sequence, 1..16.
 *   q        : bf16 bits [B][Q][H][128];  w : fp32 [B][Q][H].
 *   len      : int32 [B], one length per cache (all its queries see it).
 *   topk     : out int32 [B][Q][k];  pool, pool_len : out [B][Q][n_blocks*block], [B][Q].
 *   scores_opt : optional out fp32 [B][Q][cap].
 *   ws, ws_bytes : workspace of at least csa2_index_full_mq_workspace(...) bytes.
 * Every other argument, the rules and the status codes are csa2_index_full's.
 */
size_t csa2_index_full_mq_workspace(int32_t B, int32_t Q, int64_t cap, int32_t k, int32_t block,
                                    int32_t n_blocks);
int csa2_index_full_mq(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                       const int32_t* len, int32_t B, int32_t Q, const uint16_t* q, const float* w,
                       int32_t H, int32_t k, int32_t block, int32_t n_blocks, int32_t* topk,
                       int32_t* pool, int32_t* pool_len, float* scores_opt, void* ws, size_t ws_bytes,
                       void* stream);
/* The same with FP4 queries (csa2_index_full_fp4q's format):
 * q_codes u8 [B][Q][H][64] (16-byte aligned), q_scales u8 [B][Q][H][4]. */
int csa2_index_full_mq_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                            const int32_t* len, int32_t B, int32_t Q, const uint8_t* q_codes,
                            const uint8_t* q_scales, const float* w, int32_t H, int32_t k, int32_t block,
                            int32_t n_blocks, int32_t* topk, int32_t* pool, int32_t* pool_len, float* scores_opt,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_full_fp4q, csa2_index_pool_fp4q -- the two indexer calls with an
 * FP4 indexer query [syt-nju.github.io, "为什么读输入只激活 8B", section
 * FP4 主 KV 缓存: the indexer's query and keys were already FP4 through
 * quantisation-aware training before the main KV was].  Both score operands
 * are then MX-FP4 (E2M1 codes, one E8M0 scale per 32 dims), and the product
 * runs on gfx950's scaled FP4 matrix instruction without dequantising.
 *   q_codes  : u8 [B][H][64] E2M1 codes of the 128-dim queries (element 2i
 *              in the low nibble of byte i), 16-byte aligned;
 *   q_scales : u8 [B][H][4] E8M0 scale bytes, one per 32 dims
 *              (csa2_quantize_fp4 with group 32 and E8M0 produces both).
 * The score is the same formula with q = the dequantised query:
 *   score[b][p] = sum_h w[b][h] * max(0, deq(q[b][h]) . deq(idx K[b][p])).
 * Every other argument, the workspace, the outputs, the selection rules and
 * the status codes are those of csa2_index_full / csa2_index_pool.  This is
 * a numerics variant: the query is rounded to FP4 by the caller.
 */
int csa2_index_full_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                         const int32_t* len, int32_t B, const uint8_t* q_codes,
                         const uint8_t* q_scales, const float* w, int32_t H, int32_t k,
                         int32_t block, int32_t n_blocks, int32_t* topk, int32_t* pool,
                         int32_t* pool_len, float* scores_opt, void* ws, size_t ws_bytes,
                         void* stream);
int csa2_index_pool_fp4q(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t cap,
                         const int32_t* len, int32_t B, const int32_t* pool,
                         const int32_t* pool_len, int32_t pool_cap, const uint8_t* q_codes,
                         const uint8_t* q_scales, const float* w, int32_t H, int32_t k,
                         int32_t* topk, float* pool_scores_opt, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * csa2_sparse_attn_decode -- core attention of one CSA2 layer for one decode
 * query per sequence: the selected main-KV entries concatenated with the
 * sliding-window entries, attended by the layer's own query; FP4 is storage
 * only, rows are dequantised before the products [SY CSA2 Figure 4; SY FP4 主 KV
 * 缓存; JU 顺便算清另外三笔账 (512 + 128 positions)].
 *   rows_b = [deq(main[b][topk[b][j]]) for valid j] ++ [deq(swa[b][r]) for r < swa_len[b]]
 *   out[b][h] = softmax_j(sm_scale * q[b][h] . rows_b[j]) @ rows_b   (K = V = row)
 *   q        : bf16 bits [B][H][512].  H : 16, 32 or 64 (multiple of 16).
 *   main_codes/main_scales : main planes [B][cap][256] / [B][cap][32], format main_fmt.
 *   len      : int32 [B] valid main entries per sequence.
 *   topk     : int32 [B][k], k <= 2048 (any order; duplicates are attended twice).
 *   swa_codes/swa_scales : window planes, sequence b at row offset b*swa_stride;
 *              swa_len : int32 [B] rows used (<= swa_cap), any slot order.
 *   swa_cap  : 0..128; may be 0 (then swa pointers may be NULL).
 *   swa_fmt  : CSA2_SWA_MAIN: window rows in the main format (256 + 32 B);
 *              CSA2_SWA_FP8: FP8 window records as csa2_window_write writes
 *              them (576 + 8 B; swa_scales 8-byte aligned) [GP 4.1; GP 7].
 *   q_pos    : int64 [B] query positions, or NULL.  With positions, each
 *              query's dims 448..511 are rotated by the compressed RoPE at
 *              q_pos[b] before the products, and the output's dims 448..511
 *              are turned back by -q_pos[b] (the fused Q RoPE and output
 *              inverse RoPE of [WG 10]); the rows are read as written, i.e.
 *              rotated at their own positions by csa2_cache_write.  8-byte
 *              aligned.
 *   out      : out bf16 bits [B][H][512].
 *   lse_opt  : optional out fp32 [B][H], natural-log sum of exp(sm_scale*logits);
 *              -inf (and a zero output row) when a sequence attends no row.
 *   ws, ws_bytes : workspace of at least csa2_attn_workspace(...) bytes.
 *              Its first CSA2_ATTN_WS_COUNTER_BYTES bytes hold completion
 *              counters that must be zero before the first call (zero-fill
 *              the workspace once after allocating it); every call leaves
 *              them zero.  The rest (partial outputs, maxima, sums) needs no
 *              initial contents.  Calls sharing a workspace must be ordered
 *              on one stream; concurrent calls on one workspace race.
 *              B*H/16 must not exceed CSA2_ATTN_MAX_GROUPS.
 * One kernel on `stream`.  Below 48 sequences (or H < 64) a workgroup attends
 * one chunk of 128 or 160 row slots for 16 heads and leaves its partial
 * (unnormalised output, max, sum) in the workspace; the last chunk of each
 * (sequence, head group) to finish merges all of them exactly.  From 48
 * sequences with H = 64, a workgroup takes all heads of a sequence over a
 * range of 32-row chunks (FP8 window records: 16-row chunks) with an online
 * softmax (one range per sequence from
 * 256 sequences), and the last range of a sequence merges the others.  The chunks of one group are placed on one XCD
 * (workgroup ids congruent mod 8; gfx950 dispatches workgroup i to XCD
 * i mod 8), so the partials meet in that XCD's L2 and a relaxed counter
 * orders them; a merge that finds a chunk from another XCD writes NaN rather
 * than a wrong value.  The result is deterministic (fixed merge order; the counters only
 * decide which workgroup merges).
 */
size_t csa2_attn_workspace(int32_t B, int32_t H, int32_t k, int32_t swa_cap);
int csa2_sparse_attn_decode(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                            const uint8_t* main_scales, int64_t cap, int32_t main_fmt,
                            const int32_t* len, const int32_t* topk, int32_t k, int32_t B,
                            const uint8_t* swa_codes, const uint8_t* swa_scales,
                            int64_t swa_stride, int32_t swa_cap, const int32_t* swa_len,
                            int32_t swa_fmt, float sm_scale, const int64_t* q_pos, uint16_t* out,
                            float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_decode_mq -- csa2_sparse_attn_decode for Q queries per
 * sequence that arrive together, such as the draft positions of a
 * speculative verify block [WG 7 (DSpark: 5 parallel draft positions)], each
 * with its own index list over its sequence's cache, in one call.
 *   q        : bf16 bits [B][Q][H][512];  topk : int32 [B][Q][k];
 *   q_pos    : int64 [B][Q] or NULL;  out : bf16 bits [B][Q][H][512];
 *   lse_opt  : fp32 [B][Q][H] or NULL.
 *   main planes, len [B], the window planes (sequence b at b*swa_stride) and
 *   swa_len [B] are per sequence, as in csa2_sparse_attn_decode, and shared
 *   by the sequence's Q queries.
 *   Q        : 1..CSA2_MAX_QUERIES_PER_SEQ.
 *   ws       : at least csa2_attn_workspace(B*Q, H, k, swa_cap) bytes, as above.
 * Query row (b, i) gives exactly what csa2_sparse_attn_decode gives for a
 * batch of B*Q queries whose sequence b*Q + i holds sequence b's cache,
 * length and window; with Q = 1 this is csa2_sparse_attn_decode.  One kernel;
 * B*Q query rows choose the kernel shape as B*Q sequences would.
 * Errors: as csa2_sparse_attn_decode; Q outside 1..CSA2_MAX_QUERIES_PER_SEQ
 * or B*Q beyond int32 is CSA2_ERR_SHAPE.
 */
int csa2_sparse_attn_decode_mq(const uint16_t* q, int32_t H, int32_t Q, const uint8_t* main_codes,
                               const uint8_t* main_scales, int64_t cap, int32_t main_fmt, const int32_t* len,
                               const int32_t* topk, int32_t k, int32_t B, const uint8_t* swa_codes,
                               const uint8_t* swa_scales, int64_t swa_stride, int32_t swa_cap,
                               const int32_t* swa_len, int32_t swa_fmt, float sm_scale, const int64_t* q_pos,
                               uint16_t* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_decode_noalloc -- csa2_sparse_attn_decode for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, outputs, kernels
 * and results, without ws/ws_bytes: the partials and completion counters live
 * in a library-held device array of CSA2_ATTN_NOALLOC_SCRATCH_BYTES (32 MiB)
 * per GPU, kept until the process ends.  The call allocates nothing.
 *   Limit: csa2_attn_workspace(B, H, k, swa_cap) must not exceed
 *   CSA2_ATTN_NOALLOC_SCRATCH_BYTES (e.g. up to 96 sequences at H = 64,
 *   k = 512, swa_cap = 128), else CSA2_ERR_SCRATCH and nothing is launched.
 *   The current device must be the device of `stream` and of the buffers.
 *   The first call on a device takes the array's device address and clears
 *   its counters with a small kernel on `stream`; every call leaves them zero.
 *   All calls on one GPU share the array: calls that overlap in time (on
 *   different streams, or in graphs replayed concurrently) race.
 */
int csa2_sparse_attn_decode_noalloc(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                                    const uint8_t* main_scales, int64_t cap, int32_t main_fmt,
                                    const int32_t* len, const int32_t* topk, int32_t k, int32_t B,
                                    const uint8_t* swa_codes, const uint8_t* swa_scales,
                                    int64_t swa_stride, int32_t swa_cap, const int32_t* swa_len,
                                    int32_t swa_fmt, float sm_scale, const int64_t* q_pos, uint16_t* out,
                                    float* lse_opt, void* stream);

/*
 * Paged cache [GP 7: the cache is paged with 576-byte alignment].  The four
 * planes of all sequences live in one pool of n_rows entries (row r of each
 * plane: main codes [r][256], main scales [r][32], indexer codes [r][64],
 * indexer scales [r][4]), in pages of P = 2^page_shift entries
 * (CSA2_MIN_PAGE_SHIFT..CSA2_MAX_PAGE_SHIFT, so a page holds at least 64
 * entries).  Entry i of sequence b is pool row
 *     block_table[b * max_pages + i / P] * P + i % P,
 * block_table : int32 [B][max_pages], page ids in [0, n_rows / P) (an id
 * outside is clamped into the pool: a stale table reads a wrong row of the
 * pool, never memory outside it).  Logical capacity max_pages * P <=
 * CSA2_MAX_CACHE_ROWS; n_rows a multiple of P, at most CSA2_MAX_POOL_ROWS.
 * Positions stay logical everywhere (lengths, top-k, pool, RoPE positions);
 * the indexer calls also return the physical rows of what they select, and
 * the Reindex and attention calls gather by those rows, so each index layer
 * resolves pages once and its Reuse layers reuse the rows.
 *
 * csa2_cache_append_paged -- csa2_cache_append into a paged pool: the entry
 * of sequence b goes to logical row len[b], i.e. pool row via block_table
 * (len[b] >= max_pages * P: full).  Other arguments as csa2_cache_append.
 *
 * csa2_index_full_paged -- csa2_index_full over a paged cache (one page-table
 * read per 64-entry tile of the scoring pass).  topk, pool, pool_len as
 * csa2_index_full (logical positions); topk_rows : out int32 [B][k] and
 * pool_rows : out int32 [B][n_blocks*block], the pool rows of the same
 * entries (-1 where topk / pool hold -1).  The workspace is
 * csa2_index_full_workspace(B, max_pages * P, k, block, n_blocks).
 *
 * csa2_index_pool_rows -- csa2_index_pool gathering by physical rows:
 * pool_rows [B][pool_cap] (as csa2_index_full_paged writes them; -1 or a row
 * outside [0, n_rows) is masked) scored for the ranking, pool [B][pool_cap]
 * the same entries' logical positions for the output.  topk : out logical
 * positions, topk_rows : out their pool rows (-1 padded).  No lengths: the
 * rows carry visibility.  Workspace: csa2_index_pool_workspace.
 *
 * csa2_sparse_attn_decode_rows -- csa2_sparse_attn_decode with the selected
 * entries given as pool rows: rows [B][k] into the main planes of n_rows
 * entries (-1 or a row outside [0, n_rows) is masked; no lengths).  The
 * window arguments, outputs, workspace and status codes are those of
 * csa2_sparse_attn_decode.
 */
int csa2_cache_append_paged(const uint16_t* latent, const uint16_t* gate, int32_t B, int32_t m,
                            const float* gamma, float eps, const float* w_idx, int32_t main_fmt, int32_t rope,
                            uint8_t* main_codes, uint8_t* main_scales, uint8_t* idx_codes, uint8_t* idx_scales,
                            int64_t n_rows, const int32_t* block_table, int32_t page_shift, int32_t max_pages,
                            int32_t* len, void* state, void* stream);
int csa2_index_full_paged(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t n_rows,
                          const int32_t* block_table, int32_t page_shift, int32_t max_pages,
                          const int32_t* len, int32_t B, const uint16_t* q, const float* w, int32_t H,
                          int32_t k, int32_t block, int32_t n_blocks, int32_t* topk, int32_t* topk_rows,
                          int32_t* pool, int32_t* pool_rows, int32_t* pool_len, float* scores_opt,
                          void* ws, size_t ws_bytes, void* stream);
int csa2_index_pool_rows(const uint8_t* idx_codes, const uint8_t* idx_scales, int64_t n_rows, int32_t B,
                         const int32_t* pool, const int32_t* pool_rows, const int32_t* pool_len,
                         int32_t pool_cap, const uint16_t* q, const float* w, int32_t H, int32_t k,
                         int32_t* topk, int32_t* topk_rows, float* pool_scores_opt, void* ws, size_t ws_bytes,
                         void* stream);
int csa2_sparse_attn_decode_rows(const uint16_t* q, int32_t H, const uint8_t* main_codes,
                                 const uint8_t* main_scales, int64_t n_rows, int32_t main_fmt,
                                 const int32_t* rows, int32_t k, int32_t B, const uint8_t* swa_codes,
                                 const uint8_t* swa_scales, int64_t swa_stride, int32_t swa_cap,
                                 const int32_t* swa_len, int32_t swa_fmt, float sm_scale, const int64_t* q_pos,
                                 uint16_t* out, float* lse_opt, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
