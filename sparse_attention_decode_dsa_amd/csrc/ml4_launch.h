// Internal interface between the C-ABI shim (abi.cpp) and the kernel launchers.  Host-only
// types; every pointer is a device pointer.  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace ml4 {

struct SeqView {
  int batch, total_q, max_seq_len, max_q_per_seq;
  int lbs;    // log2(block_size)
  int mbps;   // block_table row stride
  const int32_t* seq_lens;
  const int32_t* q_start;
  const int32_t* q_pos;
  const int32_t* block_table;
};

struct IndexerLaunch {
  SeqView s;
  const void* pool;
  int64_t num_blocks;
  bool fp8;             // ML4_IDX_FP8_132 + e4m3 q; else ML4_IDX_F32 + fp32 q
  const void* q;
  const float* q_scale; // may be null
  const float* w;
  int n_heads;
  float ssmax_s;
  float* scores;
  int64_t ld;
  uint32_t* fault;
};
hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st);

struct TopkLaunch {
  SeqView s;
  const float* scores;
  int64_t ld;
  int top_k;
  int32_t* idx;
  int32_t* len;
  void* ws;
  uint32_t* fault;
};
size_t topk_ws_bytes(const SeqView& s, int top_k);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t st);

struct MlaLaunch {
  SeqView s;
  const void* pool;
  int64_t num_blocks;
  bool fp8;             // ML4_LAT_FP8_656 / ML4_LAT_BF16_1152 + bf16 q/out; else ML4_LAT_F32
  bool bf16_rows;       // ML4_LAT_BF16_1152
  bool e4m3_rows;       // ML4_LAT_E4M3_576 with E4M3 queries
  const float* q_scale; // [total_q][n_heads] (E4M3 queries)
  float kv_scale;       // per-tensor scale of the E4M3 rows
  int window;           // > 0: attend to the last `window` positions (idx / len unused)
  const void* q;
  int n_heads;
  int rope_dim;
  const int32_t* idx;
  const int32_t* len;
  int top_k;
  float softmax_scale;
  float ssmax_s;
  void* out;
  float* lse;           // may be null
  void* ws;
  uint32_t* fault;
};
size_t mla_ws_bytes(const SeqView& s, int n_heads, int top_k);
hipError_t launch_mla(const MlaLaunch& a, hipStream_t st);

struct CacheWriteLaunch {
  bool latent;          // latent rows (656-B fp8_ds_mla unless a flag below); else 132-B indexer rows
  bool bf16_rows;       // latent: 1,152-B bf16 rows
  bool e4m3_rows;       // latent: 576-B plain E4M3 rows, codes = E4M3(x / kv_scale)
  float kv_scale;       // e4m3_rows: per-tensor scale, finite and > 0
  void* pool;
  int64_t capacity;     // num_blocks * block_size rows
  const void* src;      // [n_tokens][128 | 512]
  bool bf16;            // src dtype bf16; else fp32
  const void* rope;     // [n_tokens][64] bf16 (latent with rope_dim 64), else null
  int rope_dim;
  int64_t n_tokens;
  const int64_t* slot_mapping;
  uint32_t* fault;
};
hipError_t launch_cache_write(const CacheWriteLaunch& a, hipStream_t st);

struct MergeLaunch {
  int rows, n_shards;
  int64_t ld;                 // entries per shard list
  const float* cand_scores;   // [rows][n_shards][ld]
  const int32_t* cand_pos;    // [rows][n_shards][ld]
  const int32_t* cand_len;    // [rows][n_shards]
  int top_k;
  int32_t* idx;
  int32_t* len;
  uint32_t* fault;
};
hipError_t launch_topk_merge(const MergeLaunch& a, hipStream_t st);

struct LseCombineLaunch {
  int rows, n_heads, n_shards, head_dim;
  const float* o_parts;       // [rows][n_shards][n_heads][head_dim]
  const float* lse_parts;     // [rows][n_shards][n_heads], natural log
  void* out;                  // [rows][n_heads][head_dim]
  bool out_bf16;
  float* lse;                 // [rows][n_heads] or null
};
hipError_t launch_lse_combine(const LseCombineLaunch& a, hipStream_t st);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Replaces the thread-local text that ml4_last_error() returns.
void set_last_error(const std::string& msg);

// Device address of the current device's copy of the library's fixed scratch array
// (ML4_STATIC_SCRATCH_BYTES, 256-B aligned), looked up on its first use on that device.
hipError_t static_scratch_address(void** out);

}  // namespace ml4
