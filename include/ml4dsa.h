/*
 * ml4dsa.h -- C ABI of the MI355X (gfx950) library for the DeepSeek-style sparse-attention
 * step of Mistral Large 4: DSA indexer scores -> exact top-k -> sparse MLA over the selected
 * latent rows, with NoPE, shared-indexer and KV-sharing-consumer layers.
 *
 * Pages cited (by title and section):
 *   [blog]   "vLLM 首日支持 Mistral Large 4：1T 参数 MoE 多模态模型" (best2ai.com translation of
 *            the vLLM day-0 post)
 *   [recipe] "mistralai/Mistral-Large-4-1T-A52B — vLLM serving recipe" (recipes.vllm.ai)
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every buffer,
 *     including workspace and the fault word; the library keeps no pointer after a call
 *     returns.  Work is enqueued asynchronously on `stream` (NULL = the default stream); no
 *     entry point synchronises except ml4_fault_query.
 *   - Return value: ML4_OK (0) or a negative ml4_status.  Host-side validation is
 *     default-deny [blog, ROCm implementation details › 专用解码 / default-deny: refuse and
 *     list every reason]: every argument check is evaluated, every failure is listed, one
 *     per line, in the thread-local ml4_last_error(), and nothing is launched.
 *   - Device-side problems (a block id outside the pool, a top-k entry outside [0, q_pos],
 *     a NaN score, q_pos outside [0, seq_len)) set bits in the caller's sticky fault word
 *     [blog, ROCm implementation details › Fail-stop: a sticky fault word checked after
 *     each forward] and the affected key or row is masked; kernels always run to
 *     completion.  ml4_fault_query() reads the word.
 *   - The library allocates no device memory and never calls hipMalloc/hipFree; its only
 *     device memory is the fixed scratch array of ml4_sparse_attn_layer_static.
 */
#ifndef ML4DSA_H
#define ML4DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;   /* HIP's opaque stream handle */

/* 6: the cache-write entries require 16-byte aligned source rows. */
#define ML4_ABI_VERSION 6

enum ml4_status {
  ML4_OK = 0,
  ML4_E_INVALID = -1,       /* an argument is out of its documented range       */
  ML4_E_UNSUPPORTED = -2,   /* a valid combination the library does not provide  */
  ML4_E_WORKSPACE = -3,     /* ws_bytes below ml4_workspace_bytes()              */
  ML4_E_LAUNCH = -4,        /* the HIP runtime refused a launch                  */
  ML4_E_DEVICE_FAULT = -5   /* ml4_fault_query found fault bits set              */
};

enum ml4_dtype { ML4_F32 = 0, ML4_BF16 = 1, ML4_FP8_E4M3 = 2 };

/* Indexer cache row formats.  [blog, ROCm implementation details › AITER 上的 DSA 索引器:
 * FP8 indexer keys with a single scale per key, 132 bytes per token per indexer layer] */
enum ml4_index_format {
  ML4_IDX_F32 = 0,      /* 128 x fp32 = 512 B per token; no key scale (fp32 test format)    */
  ML4_IDX_FP8_132 = 1   /* [128 x e4m3 (OCP E4M3FN)][fp32 key scale] = 132 B per token      */
};

/* Latent cache row formats.  [blog, Implementation details › 稀疏 MLA + DSA indexer (latent
 * cache in fp8_ds_mla); ROCm implementation details › FP8 潜在缓存 (656 B per token per
 * layer)]; KV LoRA rank 512 and RoPE dim 64 [blog, Highlights]. */
enum ml4_latent_format {
  ML4_LAT_F32 = 0,      /* [512 x fp32 latent][64 x fp32 RoPE] = 2,304 B (fp32 test format) */
  ML4_LAT_FP8_656 = 1,  /* [512 x e4m3][4 x fp32 scale, one per 128][64 x bf16 RoPE] = 656 B */
  ML4_LAT_BF16_1152 = 2, /* [512 x bf16][64 x bf16 RoPE] = 1,152 B ([blog] FP8 潜在缓存: the
                           uncompressed bf16 row the FP8 layouts are measured against)     */
  ML4_LAT_E4M3_576 = 3  /* [512 x e4m3][64 x e4m3 RoPE] = 576 B, value = code * kv_scale with
                           one per-tensor scale ([blog] FP8 潜在缓存: the ROCm layout)       */
};

#define ML4_IDX_DIM 128
#define ML4_KV_LORA 512
#define ML4_ROPE_DIM 64
#define ML4_IDX_ROW_FP8 132
#define ML4_LAT_ROW_FP8 656
#define ML4_MAX_TOPK 2048

enum ml4_fault_bits {
  ML4_FAULT_BLOCK_ID = 1u << 0,    /* block_table entry outside [0, num_blocks)           */
  ML4_FAULT_TOPK_INDEX = 1u << 1,  /* topk entry outside [0, q_pos] or topk_len > top_k    */
  ML4_FAULT_NAN_SCORE = 1u << 2,   /* a candidate score was NaN (ranked below -inf)        */
  ML4_FAULT_QPOS = 1u << 3,        /* q_pos outside [0, seq_len) or > max_seq_len - 1      */
  ML4_FAULT_RANGE = 1u << 4        /* fp8 MLA: a non-finite bf16 latent-query element, or a
                                      selected key's latent scale with |s| > 128 or NaN;
                                      plain-E4M3 MLA: a non-finite query scale; that row's
                                      output is unspecified                                */
};

/* A batch of requests.  [host] struct; the arrays are device memory.
 * Request b owns query rows q_start[b] .. q_start[b+1]-1; row r sees logical key positions
 * 0 .. q_pos[r] (a query sees its own key).  Logical position t of request b lives in cache
 * slot block_table[b][t / block_size] * block_size + t % block_size [blog, ROCm
 * implementation details › AITER 上的稀疏 MLA: top-k positions become global cache slots,
 * one entry per query token]. */
typedef struct {
  int32_t batch;               /* requests B >= 1                                           */
  int32_t total_q;             /* query rows = q_start[B] >= 1                              */
  int32_t max_seq_len;         /* host bound: seq_lens[b] <= max_seq_len (sizes grids)     */
  int32_t max_q_per_seq;       /* host bound: q_start[b+1] - q_start[b] <= max_q_per_seq   */
  int32_t block_size;          /* tokens per block: power of two, 16 .. 65536 (pages: 64)  */
  int32_t max_blocks_per_seq;  /* row stride of block_table, >= ceil(max_seq_len/bs)       */
  const int32_t* seq_lens;     /* [B]   cached tokens, including this step's               */
  const int32_t* q_start;      /* [B+1] query-row offsets, q_start[0] = 0                   */
  const int32_t* q_pos;        /* [total_q] absolute position of each query row            */
  const int32_t* block_table;  /* [B][max_blocks_per_seq] physical block ids               */
} ml4_seqs;

/* One layer's cache: pool = [num_blocks][block_size][row bytes of `format`], 16-B aligned. */
typedef struct {
  const void* pool;
  int64_t num_blocks;
  int32_t format;              /* ml4_index_format or ml4_latent_format                     */
} ml4_cache;

/*
 * ml4_indexer_score -- DSA indexer scores over every visible cached key.
 * [blog, Highlights (DSA sparse indexer); Implementation details › 稀疏 MLA + DSA indexer
 * (FP8 indexer cache; the indexer has its own SSMax); ROCm implementation details › AITER 上的
 * DSA 索引器 (132-B FP8 keys, one scale per key; paged decode scores and prefill scores)]
 *   scores[r][t] = m_r * ks[t] * sum_h w[r][h] * qs[r][h] * ReLU(sum_d q[r][h][d] * k[t][d])
 *   for 0 <= t <= q_pos[r];  -inf for q_pos[r] < t < max_seq_len; columns >= max_seq_len are
 *   not written.  m_r = ssmax_s * ln(q_pos[r] + 1) when ssmax_s > 0, else 1.
 *   q        [total_q][n_heads][128]: e4m3 codes (ML4_FP8_E4M3) with an ML4_IDX_FP8_132
 *            cache, or fp32 (ML4_F32) with an ML4_IDX_F32 cache; 16-B aligned.
 *   q_scale  [total_q][n_heads] fp32, or NULL (= 1).   w [total_q][n_heads] fp32.
 *   n_heads  multiple of 16, 16 .. 64.   ld_scores >= max_seq_len, multiple of 4.
 * Decode rows stream the paged cache; rows of one request share each key load (speculative
 * verify, prefill).  fp32 accumulation; the fp8 products are exact.
 */
int ml4_indexer_score(const ml4_seqs* s, const ml4_cache* idx_cache, const void* q,
                      int32_t q_dtype, const float* q_scale, const float* w, int32_t n_heads,
                      float ssmax_s, float* scores, int64_t ld_scores, uint32_t* fault,
                      hipStream_t stream);

/*
 * ml4_topk_select -- exact top-k of each row's visible scores.
 * [blog, ROCm implementation details › 专用解码 (exact top-2048); Long context › DCP (a
 * stable top-k merge; radix select over packed (score, id) candidates; top-k compaction:
 * -1 padded slots bounded by topk_length); recipe/blog: index_topk]
 *   Candidates t in [0, q_pos[r]] of scores[r][*].  Order: higher score first, then lower t;
 *   -0 == +0; NaN ranks below -inf (and sets ML4_FAULT_NAN_SCORE).
 *   topk_idx [total_q][top_k] int32: the selected positions in ascending t, then -1.
 *   topk_len [total_q] int32 = min(top_k, q_pos[r] + 1).
 *   1 <= top_k <= 2048.  ws: ml4_workspace_bytes(ML4_ENTRY_TOPK, ...) bytes: 0 when
 *   max_seq_len <= 131,072, else per-chunk candidate lists (8 bytes per position and row
 *   plus a length per 16,384 positions and row), written before they are read.
 * Integer work on the order-preserving u32 image of each fp32 score: deterministic.
 */
int ml4_topk_select(const ml4_seqs* s, const float* scores, int64_t ld_scores, int32_t top_k,
                    int32_t* topk_idx, int32_t* topk_len, void* ws, size_t ws_bytes,
                    uint32_t* fault, hipStream_t stream);

/*
 * ml4_sparse_mla_decode -- MLA attention over the selected latent rows.
 * [blog, Highlights (MLA, KV LoRA rank 512, RoPE dim 64, top 2048 keys per query);
 * Implementation details › 稀疏 MLA + DSA indexer (sparse MLA over the fp8_ds_mla latent
 * cache); › NoPE、SSMax 和 LeRoPE (NoPE = MLA with RoPE dim 0, same kernel and layout; SSMax
 * logit scaling); › 跨层 KV 共享 (a consumer layer reads its target layer's cache);
 * Long context › DCP (partial attention merged by log-sum-exp)]
 *   For row r, head h, over its valid selected positions t (topk_idx[r][0..topk_len[r])):
 *     l_t = sigma_r * (qa[r][h] . c_t + qr[r][h] . kr_t),
 *     sigma_r = softmax_scale * (ssmax_s > 0 ? ssmax_s * ln(q_pos[r] + 1) : 1),
 *     out[r][h] = sum_t softmax(l)_t * c_t   (the latent row is key and value),
 *     lse[r][h] = natural-log log-sum-exp of l (or -inf when topk_len[r] == 0, out = 0).
 *   kv       the latent cache to read: the layer's own, or the target's for a consumer;
 *            ML4_LAT_FP8_656, ML4_LAT_BF16_1152 or ML4_LAT_F32 (an ML4_LAT_E4M3_576 cache
 *            carries scales and goes through ml4_sparse_mla_decode_e4m3).
 *   q        [total_q][n_heads][512 + rope_dim]: bf16 (ML4_BF16) with ML4_LAT_FP8_656 and
 *            ML4_LAT_BF16_1152, fp32 with ML4_LAT_F32.   n_heads: multiple of 16, 16 .. 128.
 *            rope_dim: 64, or 0 (NoPE: the RoPE bytes are never read).
 *   out      [total_q][n_heads][512]: bf16 (ML4_BF16) for the fp8 and bf16 caches, fp32 for
 *            the fp32 cache.   lse: fp32 [total_q][n_heads] or NULL.
 *   ws       ml4_workspace_bytes(ML4_ENTRY_MLA, ...) bytes (split-K partials; may be 0).
 * Dequantisation of e4m3 codes is exact.  With the fp8 cache the QK products (latent and
 * RoPE) run on bf16 MFMA with the query as given (e4m3 codes are bf16 values; a non-finite
 * query element raises ML4_FAULT_RANGE) and PV on fp16 MFMA, all with fp32 accumulation;
 * the softmax weights are rounded to fp16 after the running-max shift.
 * With the bf16 cache QK and the RoPE product run on bf16 MFMA with the query as given and
 * PV on fp16 MFMA (the latent values must lie within the fp16 range).
 */
int ml4_sparse_mla_decode(const ml4_seqs* s, const ml4_cache* kv, const void* q,
                          int32_t q_dtype, int32_t n_heads, int32_t rope_dim,
                          const int32_t* topk_idx, const int32_t* topk_len, int32_t top_k,
                          float softmax_scale, float ssmax_s, void* out, int32_t out_dtype,
                          float* lse, void* ws, size_t ws_bytes, uint32_t* fault,
                          hipStream_t stream);

/*
 * ml4_sparse_mla_decode_e4m3 -- ml4_sparse_mla_decode over plain E4M3 latent rows with FP8
 * queries.  [blog, ROCm implementation details › FP8 潜在缓存 (all 576 latent dims stored as
 * E4M3 with one per-tensor scale, 576 B per token per layer; the queries are quantised to FP8
 * as well, so QK runs FP8 x FP8)]
 *   The formula of ml4_sparse_mla_decode on the decoded values
 *     c_t|kr_t = e4m3(code) * kv_scale,   qa|qr[r][h] = e4m3(q code) * q_scale[r][h].
 *   kv       an ML4_LAT_E4M3_576 cache.   kv_scale: finite, > 0.
 *   q        [total_q][n_heads][512 + rope_dim] e4m3 codes (OCP E4M3FN), 16-B aligned.
 *   q_scale  [total_q][n_heads] fp32 (a non-finite scale raises ML4_FAULT_RANGE).
 *   out      [total_q][n_heads][512] bf16 (out_dtype ML4_BF16).   lse: fp32 or NULL.
 *   Other arguments, workspace and fault bits as for ml4_sparse_mla_decode.
 * QK runs on FP8 MFMA with fp32 accumulation (products exact; the hardware's 128-term sum may
 * drop low-order bits of small products); PV decodes V exactly to fp16 and runs on fp16 MFMA
 * with the softmax weights rounded to fp16; kv_scale multiplies the normalised output.
 */
int ml4_sparse_mla_decode_e4m3(const ml4_seqs* s, const ml4_cache* kv, float kv_scale,
                               const uint8_t* q, const float* q_scale, int32_t n_heads,
                               int32_t rope_dim, const int32_t* topk_idx,
                               const int32_t* topk_len, int32_t top_k, float softmax_scale,
                               float ssmax_s, void* out, int32_t out_dtype, float* lse,
                               void* ws, size_t ws_bytes, uint32_t* fault,
                               hipStream_t stream);

/*
 * ml4_window_mla_decode -- MLA over the last `window` positions of each row (a sliding
 * window, no indexer), on the same kernel.  [blog, Long context (DSpark draft layers attend
 * to a 2,048-token sliding window over a bf16 KV cache)]
 *   Row r attends to positions max(0, q_pos[r] - window + 1) .. q_pos[r] with the formula of
 *   ml4_sparse_mla_decode.  kv: ML4_LAT_BF16_1152 or ML4_LAT_FP8_656.  1 <= window <= 2048.
 *   ws: ml4_workspace_bytes(ML4_ENTRY_MLA, s, n_heads, window) bytes.
 *   With ML4_LAT_BF16_1152 the latent values must lie within the fp16 range (PV runs on
 *   fp16 MFMA); QK and the RoPE part run on bf16 MFMA with the query as given.
 */
int ml4_window_mla_decode(const ml4_seqs* s, const ml4_cache* kv, const void* q,
                          int32_t q_dtype, int32_t n_heads, int32_t rope_dim, int32_t window,
                          float softmax_scale, float ssmax_s, void* out, int32_t out_dtype,
                          float* lse, void* ws, size_t ws_bytes, uint32_t* fault,
                          hipStream_t stream);

/* One layer's role.  [blog, Model architecture (every 4th layer NoPE; 28 layers reuse the
 * nearest preceding indexer layer's top-k; NoPE layers 39-71 read layer 35's latent KV);
 * 跨层 KV 共享 (kv_sharing_target_layer_name); 稀疏 MLA + DSA indexer (shared indexer layers
 * reuse the top-k)] */
typedef struct {
  int32_t layer;                    /* this layer's index, < n_layers                       */
  int32_t kv_sharing_target_layer;  /* -1: own latent cache; else an earlier layer whose
                                       cache this consumer reads (no write)                 */
  int32_t topk_source_layer;        /* -1: run own indexer; else an earlier indexer layer
                                       whose top-k is reused bit for bit                    */
  int32_t rope_dim;                 /* 64, or 0 for NoPE                                     */
  int32_t top_k;                    /* index_topk, 1 .. 2048                                 */
  int32_t idx_heads;                /* indexer heads (multiple of 16, 16 .. 64)              */
  int32_t mla_heads;                /* MLA heads (multiple of 16, 16 .. 128)                 */
  float softmax_scale;              /* e.g. 1/sqrt(512 + rope_dim)                           */
  float ssmax_s;                    /* MLA SSMax s (<= 0: off)                               */
  float idx_ssmax_s;                /* indexer SSMax s (<= 0: off)                           */
} ml4_layer;

/*
 * ml4_sparse_attn_layer -- one layer's indexer -> top-k -> sparse MLA in one call, no host
 * synchronisation.  [blog, ROCm implementation details › 专用解码 (the whole indexer, exact
 * top-2048 and sparse MLA inside one launch per layer, with NoPE, KV-sharing and
 * index-sharing layers)]
 *   layers: [host] array of n_layers descriptors, indexed by layer (layers[i].layer == i
 *   for this layer and every layer it names); the call runs layer `layer`.
 *   lat_caches, idx_caches: [host] arrays of n_layers caches, indexed by layer.
 *   topk_bufs, topk_lens: [host] arrays of n_layers device pointers, indexed by layer.
 *   An indexer layer (topk_source_layer < 0) scores idx_caches[layer], selects, and writes
 *   topk_bufs[layer] ([total_q][top_k]) / topk_lens[layer]; a shared-indexer layer reads
 *   topk_bufs[topk_source_layer] and runs no indexer.  The attention reads
 *   lat_caches[kv_sharing_target_layer >= 0 ? kv_sharing_target_layer : layer].
 *   Layer roles are validated from the descriptors [blog, 跨层 KV 共享; Model architecture]:
 *   the KV-sharing target must own its cache (its own kv_sharing_target_layer is -1: no
 *   chains); the top-k source must run its own indexer (its topk_source_layer is -1) and
 *   have the same top_k (the row stride of the shared buffer).  Both must be earlier layers.
 *   q_idx/q_idx_scale/w_idx as in ml4_indexer_score (ignored for a shared-indexer layer);
 *   q_mla/out/lse as in ml4_sparse_mla_decode.
 *   ws: ml4_workspace_bytes(ML4_ENTRY_LAYER, s, mla_heads, top_k) bytes (holds the scores).
 */
int ml4_sparse_attn_layer(const ml4_layer* layers, int32_t layer, const ml4_seqs* s,
                          const ml4_cache* lat_caches, const ml4_cache* idx_caches,
                          int32_t n_layers, const void* q_idx, int32_t q_idx_dtype,
                          const float* q_idx_scale, const float* w_idx, const void* q_mla,
                          int32_t q_mla_dtype, int32_t* const* topk_bufs,
                          int32_t* const* topk_lens, void* out, int32_t out_dtype, float* lse,
                          void* ws, size_t ws_bytes, uint32_t* fault, hipStream_t stream);

/*
 * ml4_sparse_attn_layer_static -- ml4_sparse_attn_layer without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It allocates nothing: the scratch (scores,
 * top-k candidate lists, split-MLA partials) is one fixed device array of
 * ML4_STATIC_SCRATCH_BYTES inside the library, which each GPU the library runs on holds
 * from the library's first use on it until the process ends.
 *   Arguments, results, validation and fault bits as ml4_sparse_attn_layer.
 *   A batch whose ml4_workspace_bytes(ML4_ENTRY_LAYER, ...) exceeds ML4_STATIC_SCRATCH_BYTES
 *   is refused with ML4_E_UNSUPPORTED (nothing launched); 64 MiB holds the scores of
 *   256 query rows at 65,536 positions, or the scores and top-k lists (12 bytes per
 *   position) of one row at up to 4M positions.
 *   Every call on one GPU uses that GPU's one array: calls that may overlap in time on the
 *   same GPU (other streams, other host threads) race and must be ordered by the caller.
 */
#define ML4_STATIC_SCRATCH_BYTES (64u << 20)
int ml4_sparse_attn_layer_static(const ml4_layer* layers, int32_t layer, const ml4_seqs* s,
                                 const ml4_cache* lat_caches, const ml4_cache* idx_caches,
                                 int32_t n_layers, const void* q_idx, int32_t q_idx_dtype,
                                 const float* q_idx_scale, const float* w_idx,
                                 const void* q_mla, int32_t q_mla_dtype,
                                 int32_t* const* topk_bufs, int32_t* const* topk_lens,
                                 void* out, int32_t out_dtype, float* lse, uint32_t* fault,
                                 hipStream_t stream);

/*
 * ml4_index_cache_write / ml4_latent_cache_write -- quantise and pack new tokens into the
 * paged caches the path reads (the step before it; a KV-sharing consumer layer calls
 * neither).  [blog, ROCm implementation details › AITER 上的 DSA 索引器 (an FP8 indexer key
 * with one scale per key, 132 B per token); › FP8 潜在缓存 (fp8_ds_mla: 512 FP8 values with
 * four per-128 scales and 64 bf16 RoPE values, 656 B per token)]
 *   Quantiser, per scale group (the whole 128-dim key; each 128 latent values):
 *     scale = amax / 448,  code = E4M3(x / scale) rounded to nearest even and clamped to
 *     +-448, in binary32; an all-zero group stores scale 0 and zero codes.
 *   cache        ML4_IDX_FP8_132 (index), ML4_LAT_FP8_656 or ML4_LAT_BF16_1152 (latent; the
 *                bf16 row takes the latents rounded to nearest even and the RoPE bits as
 *                given); rows are addressed as pool + slot * row_bytes with
 *                0 <= slot < num_blocks * block_size and written through cache->pool (which
 *                the write entries treat as writable).  ML4_LAT_E4M3_576 goes through
 *                ml4_latent_cache_write_e4m3.
 *   block_size   tokens per block (power of two, 16 .. 65536).
 *   k / c        [n_tokens][128] / [n_tokens][512], BF16 or F32 (src_dtype), 16-byte aligned
 *                (rows are read as 16-byte vectors).
 *   k_rope       [n_tokens][64] bf16 with rope_dim 64; NULL with rope_dim 0 (NoPE: the RoPE
 *                bytes of the row are left untouched).
 *   slot_mapping [n_tokens] int64: destination slot = block_id * block_size + offset;
 *                a negative slot skips that token (padding).
 *   n_tokens     >= 0 (0: nothing is launched).
 *   Device faults: a slot >= num_blocks * block_size sets ML4_FAULT_BLOCK_ID and skips
 *   the token; a non-finite input value sets ML4_FAULT_RANGE (that row is unspecified).
 */
int ml4_index_cache_write(const ml4_cache* idx_cache, int32_t block_size, const void* k,
                          int32_t src_dtype, int64_t n_tokens, const int64_t* slot_mapping,
                          uint32_t* fault, hipStream_t stream);
int ml4_latent_cache_write(const ml4_cache* lat_cache, int32_t block_size, const void* c,
                           int32_t src_dtype, const void* k_rope, int32_t rope_dim,
                           int64_t n_tokens, const int64_t* slot_mapping, uint32_t* fault,
                           hipStream_t stream);

/*
 * ml4_latent_cache_write_e4m3 -- ml4_latent_cache_write into plain E4M3 rows with one
 * per-tensor scale (the second latent layout read by ml4_sparse_mla_decode_e4m3).
 * [blog, ROCm implementation details › FP8 潜在缓存 (all 576 dims in E4M3 with a per-tensor
 * scale, 576 B per token)]
 *   Row: 512 latent codes then 64 RoPE codes, code = E4M3(x / kv_scale) rounded to nearest
 *   even and clamped to +-448, in binary32; values beyond 448 * kv_scale saturate.
 *   cache        ML4_LAT_E4M3_576.
 *   kv_scale     the per-tensor scale the reader multiplies by; finite and > 0, else
 *                ML4_E_INVALID.
 *   k_rope       [n_tokens][64] bf16 with rope_dim 64 (quantised with kv_scale); NULL with
 *                rope_dim 0 (the RoPE codes of the row are left untouched).
 *   Other arguments, errors and device faults as ml4_latent_cache_write; a non-finite
 *   latent or RoPE value sets ML4_FAULT_RANGE (that row is unspecified).
 */
int ml4_latent_cache_write_e4m3(const ml4_cache* lat_cache, int32_t block_size, const void* c,
                                int32_t src_dtype, const void* k_rope, int32_t rope_dim,
                                float kv_scale, int64_t n_tokens, const int64_t* slot_mapping,
                                uint32_t* fault, hipStream_t stream);

/*
 * ml4_topk_merge -- exact top-k over the union of per-shard candidate lists, for context
 * split across shards (devices or chunks of one long row).  [blog, Long context › DCP (each
 * shard keeps its own top-2048; a stable top-k merge over (score, position) pairs; radix
 * select over packed candidates)]
 *   cand_scores [rows][n_shards][ld_cand] fp32, cand_pos [rows][n_shards][ld_cand] int32
 *   (distinct positions >= 0 within a row), cand_len [rows][n_shards] (entries past it are
 *   ignored).  n_shards * ld_cand <= 16384, 1 <= top_k <= 2048.
 *   Order as ml4_topk_select (score descending, -0 == +0, NaN lowest and reported, equal
 *   scores lower position first); output ascending positions, -1 padded, topk_len =
 *   min(top_k, number of candidates).  A length outside [0, ld_cand] or a negative
 *   position sets ML4_FAULT_TOPK_INDEX (the entry is skipped).
 *
 * ml4_lse_combine -- merge partial attentions over disjoint key sets by their log-sum-exp.
 *   [blog, Long context › DCP (partial outputs merged through their LSE)]
 *   o_parts [rows][n_shards][n_heads][head_dim] fp32, lse_parts [rows][n_shards][n_heads]
 *   (natural log; -inf = the shard saw no key): out[r][h] = sum_s e^(lse_s - M) o_s /
 *   sum_s e^(lse_s - M), lse = M + ln sum_s e^(lse_s - M), M = max_s lse_s (out 0 and lse
 *   -inf when every shard is empty).  out [rows][n_heads][head_dim] BF16 or F32; lse
 *   [rows][n_heads] fp32 or NULL.  head_dim 1 .. 4096.
 */
int ml4_topk_merge(int32_t rows, int32_t n_shards, const float* cand_scores,
                   const int32_t* cand_pos, const int32_t* cand_len, int64_t ld_cand,
                   int32_t top_k, int32_t* topk_idx, int32_t* topk_len, uint32_t* fault,
                   hipStream_t stream);
int ml4_lse_combine(int32_t rows, int32_t n_heads, int32_t n_shards, int32_t head_dim,
                    const float* o_parts, const float* lse_parts, void* out, int32_t out_dtype,
                    float* lse, hipStream_t stream);

/*
 * Measurement probes (not part of the attention path): the rates a plain streaming read
 * and back-to-back independent MFMAs reach on this GPU, against which the kernels above
 * are also measured.  ml4_probe_read reads `bytes` (a multiple of 16, 16-B aligned) of
 * `buf` once; ml4_probe_mfma runs 256 * 8 * 4 work-groups of 4 waves, each wave issuing
 * 16 * iters MFMAs: kind 0 = v_mfma_f32_16x16x32_f16 (16,384 FLOP each), kind 1 =
 * v_mfma_scale_f32_16x16x128_f8f6f4 on E4M3 (65,536 FLOP each).  `sink` is a device buffer
 * of at least 8192 floats the kernels may write.  Return 0, -1 (invalid argument) or -4
 * (launch refused); asynchronous on `stream`.
 */
int ml4_probe_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);
int ml4_probe_mfma(int32_t kind, int32_t iters, float* sink, hipStream_t stream);

enum ml4_entry { ML4_ENTRY_TOPK = 1, ML4_ENTRY_MLA = 2, ML4_ENTRY_LAYER = 3 };

/* Workspace bytes an entry point needs for this batch (256-B aligned start required).
 * n_heads = MLA heads; top_k as passed to the entry.  [host] s. */
size_t ml4_workspace_bytes(int32_t entry, const ml4_seqs* s, int32_t n_heads, int32_t top_k);

/* Thread-local text of the last failure: one line per failed check.  Never NULL. */
const char* ml4_last_error(void);

/* Copies the fault word to *bits [host] after synchronising `stream`; returns ML4_OK when
 * no bit is set, ML4_E_DEVICE_FAULT otherwise.  The only synchronising call. */
int ml4_fault_query(const uint32_t* fault, uint32_t* bits, hipStream_t stream);

/* ML4_ABI_VERSION of the loaded library. */
int ml4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ML4DSA_H */
