// C-ABI shim: default-deny argument validation, workspace carving and kernel dispatch.
//
// Every check of an entry point is evaluated; each failure adds one line to the
// thread-local error text and nothing is launched [page "vLLM 首日支持 Mistral Large 4"
// (best2ai.com), ROCm implementation details › 专用解码: the path refuses unsupported
// deployments at start-up with an error that lists every reason].
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "ml4_launch.h"
#include "ml4dsa.h"

namespace {

thread_local std::string g_last_error;

struct Checks {
  std::vector<std::string> invalid, unsupported, workspace;
  void bad(bool cond, const char* what) { if (cond) invalid.emplace_back(what); }
  void unsup(bool cond, const char* what) { if (cond) unsupported.emplace_back(what); }
  void ws(bool cond, const std::string& what) { if (cond) workspace.push_back(what); }
  int finish(const char* entry) {
    std::string msg;
    auto add = [&](const std::vector<std::string>& v, const char* kind) {
      for (const auto& m : v) msg += std::string(entry) + ": " + kind + ": " + m + "\n";
    };
    add(invalid, "invalid");
    add(unsupported, "unsupported");
    add(workspace, "workspace");
    g_last_error = msg;
    if (!invalid.empty()) return ML4_E_INVALID;
    if (!unsupported.empty()) return ML4_E_UNSUPPORTED;
    if (!workspace.empty()) return ML4_E_WORKSPACE;
    return ML4_OK;
  }
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
int ilog2(int v) { int l = 0; while ((1 << l) < v) ++l; return l; }

constexpr int kMaxSeqLen = 1 << 24;

void check_seqs(Checks& c, const ml4_seqs* s) {
  c.bad(s == nullptr, "seqs is NULL");
  if (!s) return;
  c.bad(s->batch < 1, "seqs.batch must be >= 1");
  c.bad(s->total_q < 1, "seqs.total_q must be >= 1");
  c.bad(s->max_seq_len < 1, "seqs.max_seq_len must be >= 1");
  c.unsup(s->max_seq_len > kMaxSeqLen, "seqs.max_seq_len above 16,777,216");
  c.bad(s->max_q_per_seq < 1, "seqs.max_q_per_seq must be >= 1");
  c.bad(s->max_q_per_seq > s->total_q, "seqs.max_q_per_seq exceeds total_q");
  c.bad(!pow2(s->block_size), "seqs.block_size must be a power of two");
  c.unsup(pow2(s->block_size) && (s->block_size < 16 || s->block_size > 65536),
          "seqs.block_size outside 16 .. 65536");
  if (pow2(s->block_size) && s->max_seq_len >= 1)
    c.bad((int64_t)s->max_blocks_per_seq * s->block_size < s->max_seq_len,
          "seqs.max_blocks_per_seq * block_size < max_seq_len");
  c.bad(!s->seq_lens || !s->q_start || !s->q_pos || !s->block_table,
        "seqs arrays (seq_lens, q_start, q_pos, block_table) must be non-NULL");
  c.bad(!aligned(s->seq_lens, 4) || !aligned(s->q_start, 4) || !aligned(s->q_pos, 4) ||
            !aligned(s->block_table, 4),
        "seqs arrays must be 4-byte aligned");
}

ml4::SeqView view(const ml4_seqs* s) {
  ml4::SeqView v{};
  v.batch = s->batch;
  v.total_q = s->total_q;
  v.max_seq_len = s->max_seq_len;
  v.max_q_per_seq = s->max_q_per_seq;
  v.lbs = ilog2(s->block_size);
  v.mbps = s->max_blocks_per_seq;
  v.seq_lens = s->seq_lens;
  v.q_start = s->q_start;
  v.q_pos = s->q_pos;
  v.block_table = s->block_table;
  return v;
}

void check_cache(Checks& c, const ml4_cache* k, bool index, const char* name) {
  std::string n(name);
  if (!k) { c.invalid.push_back(n + " is NULL"); return; }
  if (!k->pool) c.invalid.push_back(n + ".pool is NULL");
  if (!aligned(k->pool, 16)) c.invalid.push_back(n + ".pool must be 16-byte aligned");
  if (k->num_blocks < 1) c.invalid.push_back(n + ".num_blocks must be >= 1");
  if (index && k->format != ML4_IDX_F32 && k->format != ML4_IDX_FP8_132)
    c.invalid.push_back(n + ".format is not an ml4_index_format");
  if (!index && k->format != ML4_LAT_F32 && k->format != ML4_LAT_FP8_656 &&
      k->format != ML4_LAT_BF16_1152 && k->format != ML4_LAT_E4M3_576)
    c.invalid.push_back(n + ".format is not an ml4_latent_format");
}

std::string bytes_msg(const char* what, size_t need, size_t have) {
  char buf[160];
  snprintf(buf, sizeof buf, "%s needs %zu bytes, %zu given", what, need, have);
  return buf;
}

int launch_status(hipError_t e, const char* entry) {
  if (e == hipSuccess) return ML4_OK;
  g_last_error = std::string(entry) + ": launch: " + hipGetErrorString(e) + "\n";
  return ML4_E_LAUNCH;
}

size_t layer_scores_bytes(const ml4_seqs* s) {
  const size_t ld = ml4::align_up((size_t)s->max_seq_len, 4);
  return ml4::align_up((size_t)s->total_q * ld * sizeof(float), 256);
}

// ---- per-entry validation (shared by the fused entry) ----
void check_scores(Checks& c, const ml4_seqs* s, const float* scores, int64_t ld) {
  c.bad(!scores, "scores is NULL");
  c.bad(!aligned(scores, 16), "scores must be 16-byte aligned");
  if (s) c.bad(ld < s->max_seq_len, "ld_scores < max_seq_len");
  c.bad(ld % 4 != 0, "ld_scores must be a multiple of 4");
}

void check_indexer(Checks& c, const ml4_cache* ic, const void* q, int32_t q_dtype,
                   const float* w, int32_t n_heads, float ssmax_s) {
  check_cache(c, ic, true, "idx_cache");
  c.bad(!q, "q is NULL");
  c.bad(!aligned(q, 16), "q must be 16-byte aligned");
  c.bad(!w, "w is NULL");
  if (ic) {
    c.bad(ic->format == ML4_IDX_FP8_132 && q_dtype != ML4_FP8_E4M3,
          "an ML4_IDX_FP8_132 cache needs ML4_FP8_E4M3 queries");
    c.bad(ic->format == ML4_IDX_F32 && q_dtype != ML4_F32,
          "an ML4_IDX_F32 cache needs ML4_F32 queries");
  }
  c.unsup(n_heads < 16 || n_heads > 64 || n_heads % 16 != 0,
          "n_heads must be a multiple of 16 in 16 .. 64");
  c.bad(!std::isfinite(ssmax_s), "ssmax_s must be finite");
}

void check_topk(Checks& c, int32_t top_k, const int32_t* idx, const int32_t* len) {
  c.bad(top_k < 1, "top_k must be >= 1");
  c.unsup(top_k > ML4_MAX_TOPK, "top_k above 2048");
  c.bad(!idx || !len, "topk_idx and topk_len must be non-NULL");
}

void check_mla(Checks& c, const ml4_cache* kv, const void* q, int32_t q_dtype, int32_t n_heads,
               int32_t rope_dim, const int32_t* idx, const int32_t* len, int32_t top_k,
               float softmax_scale, float ssmax_s, const void* out, int32_t out_dtype,
               int32_t window = 0) {
  check_cache(c, kv, false, "kv");
  c.bad(!q, "q is NULL");
  c.bad(!aligned(q, 16), "q must be 16-byte aligned");
  if (kv) {
    const bool rows16 = kv->format == ML4_LAT_FP8_656 || kv->format == ML4_LAT_BF16_1152;
    c.bad(rows16 && q_dtype != ML4_BF16,
          "an ML4_LAT_FP8_656 / ML4_LAT_BF16_1152 cache needs ML4_BF16 queries");
    c.bad(rows16 && out_dtype != ML4_BF16,
          "an ML4_LAT_FP8_656 / ML4_LAT_BF16_1152 cache writes ML4_BF16 outputs");
    c.bad(kv->format == ML4_LAT_F32 && (q_dtype != ML4_F32 || out_dtype != ML4_F32),
          "an ML4_LAT_F32 cache needs ML4_F32 queries and outputs");
    c.bad(kv->format == ML4_LAT_E4M3_576 && (q_dtype != ML4_FP8_E4M3 || out_dtype != ML4_BF16),
          "an ML4_LAT_E4M3_576 cache needs ML4_FP8_E4M3 queries and ML4_BF16 outputs");
  }
  c.unsup(n_heads < 16 || n_heads > 128 || n_heads % 16 != 0,
          "n_heads must be a multiple of 16 in 16 .. 128");
  c.unsup(rope_dim != 0 && rope_dim != ML4_ROPE_DIM, "rope_dim must be 64 or 0 (NoPE)");
  c.bad(window == 0 && (!idx || !len), "topk_idx and topk_len must be non-NULL");
  c.unsup(window > 0 && kv && (kv->format == ML4_LAT_F32 || kv->format == ML4_LAT_E4M3_576),
          "window attention needs an ML4_LAT_FP8_656 or ML4_LAT_BF16_1152 cache");
  c.bad(top_k < 1, "top_k must be >= 1");
  c.unsup(top_k > ML4_MAX_TOPK, "top_k above 2048");
  c.bad(!(softmax_scale > 0.f) || !std::isfinite(softmax_scale),
        "softmax_scale must be finite and > 0");
  c.bad(!std::isfinite(ssmax_s), "ssmax_s must be finite");
  c.bad(!out, "out is NULL");
  c.bad(!aligned(out, 16), "out must be 16-byte aligned");
}

}  // namespace

namespace ml4 {
void set_last_error(const std::string& msg) { g_last_error = msg; }
}  // namespace ml4

extern "C" {

int ml4_abi_version(void) { return ML4_ABI_VERSION; }

const char* ml4_last_error(void) { return g_last_error.c_str(); }

size_t ml4_workspace_bytes(int32_t entry, const ml4_seqs* s, int32_t n_heads, int32_t top_k) {
  if (!s || s->total_q < 1 || s->max_seq_len < 1 || !pow2(s->block_size)) return 0;
  const ml4::SeqView v = view(s);
  const size_t tk = ml4::align_up(ml4::topk_ws_bytes(v, top_k), 256);
  const size_t ml = ml4::align_up(ml4::mla_ws_bytes(v, n_heads, top_k), 256);
  switch (entry) {
    case ML4_ENTRY_TOPK: return tk;
    case ML4_ENTRY_MLA: return ml;
    case ML4_ENTRY_LAYER: return layer_scores_bytes(s) + tk + ml;
    default: return 0;
  }
}

int ml4_indexer_score(const ml4_seqs* s, const ml4_cache* idx_cache, const void* q,
                      int32_t q_dtype, const float* q_scale, const float* w, int32_t n_heads,
                      float ssmax_s, float* scores, int64_t ld_scores, uint32_t* fault,
                      hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  check_indexer(c, idx_cache, q, q_dtype, w, n_heads, ssmax_s);
  check_scores(c, s, scores, ld_scores);
  if (int rc = c.finish("ml4_indexer_score")) return rc;
  ml4::IndexerLaunch a{};
  a.s = view(s);
  a.pool = idx_cache->pool;
  a.num_blocks = idx_cache->num_blocks;
  a.fp8 = idx_cache->format == ML4_IDX_FP8_132;
  a.q = q;
  a.q_scale = q_scale;
  a.w = w;
  a.n_heads = n_heads;
  a.ssmax_s = ssmax_s;
  a.scores = scores;
  a.ld = ld_scores;
  a.fault = fault;
  return launch_status(ml4::launch_indexer(a, stream), "ml4_indexer_score");
}

int ml4_topk_select(const ml4_seqs* s, const float* scores, int64_t ld_scores, int32_t top_k,
                    int32_t* topk_idx, int32_t* topk_len, void* ws, size_t ws_bytes,
                    uint32_t* fault, hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  check_scores(c, s, scores, ld_scores);
  check_topk(c, top_k, topk_idx, topk_len);
  if (c.invalid.empty() && c.unsupported.empty()) {
    const size_t need = ml4_workspace_bytes(ML4_ENTRY_TOPK, s, 0, top_k);
    c.ws(ws_bytes < need, bytes_msg("top-k workspace", need, ws_bytes));
    c.ws(need && (!ws || !aligned(ws, 256)), "workspace must be non-NULL and 256-byte aligned");
  }
  if (int rc = c.finish("ml4_topk_select")) return rc;
  ml4::TopkLaunch a{};
  a.s = view(s);
  a.scores = scores;
  a.ld = ld_scores;
  a.top_k = top_k;
  a.idx = topk_idx;
  a.len = topk_len;
  a.ws = ws;
  a.fault = fault;
  return launch_status(ml4::launch_topk(a, stream), "ml4_topk_select");
}

int ml4_sparse_mla_decode(const ml4_seqs* s, const ml4_cache* kv, const void* q,
                          int32_t q_dtype, int32_t n_heads, int32_t rope_dim,
                          const int32_t* topk_idx, const int32_t* topk_len, int32_t top_k,
                          float softmax_scale, float ssmax_s, void* out, int32_t out_dtype,
                          float* lse, void* ws, size_t ws_bytes, uint32_t* fault,
                          hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  check_mla(c, kv, q, q_dtype, n_heads, rope_dim, topk_idx, topk_len, top_k, softmax_scale,
            ssmax_s, out, out_dtype);
  c.bad(kv && kv->format == ML4_LAT_E4M3_576,
        "an ML4_LAT_E4M3_576 cache carries scales: use ml4_sparse_mla_decode_e4m3");
  if (c.invalid.empty() && c.unsupported.empty()) {
    const size_t need = ml4_workspace_bytes(ML4_ENTRY_MLA, s, n_heads, top_k);
    c.ws(ws_bytes < need, bytes_msg("sparse-MLA workspace", need, ws_bytes));
    c.ws(need && (!ws || !aligned(ws, 256)), "workspace must be non-NULL and 256-byte aligned");
  }
  if (int rc = c.finish("ml4_sparse_mla_decode")) return rc;
  ml4::MlaLaunch a{};
  a.s = view(s);
  a.pool = kv->pool;
  a.num_blocks = kv->num_blocks;
  a.fp8 = kv->format != ML4_LAT_F32;
  a.bf16_rows = kv->format == ML4_LAT_BF16_1152;
  a.q = q;
  a.n_heads = n_heads;
  a.rope_dim = rope_dim;
  a.idx = topk_idx;
  a.len = topk_len;
  a.top_k = top_k;
  a.softmax_scale = softmax_scale;
  a.ssmax_s = ssmax_s;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.fault = fault;
  return launch_status(ml4::launch_mla(a, stream), "ml4_sparse_mla_decode");
}

int ml4_sparse_mla_decode_e4m3(const ml4_seqs* s, const ml4_cache* kv, float kv_scale,
                               const uint8_t* q, const float* q_scale, int32_t n_heads,
                               int32_t rope_dim, const int32_t* topk_idx,
                               const int32_t* topk_len, int32_t top_k, float softmax_scale,
                               float ssmax_s, void* out, int32_t out_dtype, float* lse,
                               void* ws, size_t ws_bytes, uint32_t* fault,
                               hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  check_mla(c, kv, q, ML4_FP8_E4M3, n_heads, rope_dim, topk_idx, topk_len, top_k,
            softmax_scale, ssmax_s, out, out_dtype);
  c.bad(kv && kv->format != ML4_LAT_E4M3_576, "kv.format must be ML4_LAT_E4M3_576");
  c.bad(!(kv_scale > 0.f) || !std::isfinite(kv_scale), "kv_scale must be finite and > 0");
  c.bad(!q_scale, "q_scale is NULL");
  c.bad(!aligned(q_scale, 4), "q_scale must be 4-byte aligned");
  if (c.invalid.empty() && c.unsupported.empty()) {
    const size_t need = ml4_workspace_bytes(ML4_ENTRY_MLA, s, n_heads, top_k);
    c.ws(ws_bytes < need, bytes_msg("sparse-MLA workspace", need, ws_bytes));
    c.ws(need && (!ws || !aligned(ws, 256)), "workspace must be non-NULL and 256-byte aligned");
  }
  if (int rc = c.finish("ml4_sparse_mla_decode_e4m3")) return rc;
  ml4::MlaLaunch a{};
  a.s = view(s);
  a.pool = kv->pool;
  a.num_blocks = kv->num_blocks;
  a.fp8 = true;
  a.e4m3_rows = true;
  a.q_scale = q_scale;
  a.kv_scale = kv_scale;
  a.q = q;
  a.n_heads = n_heads;
  a.rope_dim = rope_dim;
  a.idx = topk_idx;
  a.len = topk_len;
  a.top_k = top_k;
  a.softmax_scale = softmax_scale;
  a.ssmax_s = ssmax_s;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.fault = fault;
  return launch_status(ml4::launch_mla(a, stream), "ml4_sparse_mla_decode_e4m3");
}

int ml4_window_mla_decode(const ml4_seqs* s, const ml4_cache* kv, const void* q,
                          int32_t q_dtype, int32_t n_heads, int32_t rope_dim, int32_t window,
                          float softmax_scale, float ssmax_s, void* out, int32_t out_dtype,
                          float* lse, void* ws, size_t ws_bytes, uint32_t* fault,
                          hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  c.bad(window < 1, "window must be >= 1");
  check_mla(c, kv, q, q_dtype, n_heads, rope_dim, nullptr, nullptr, std::max(window, 1),
            softmax_scale, ssmax_s, out, out_dtype, std::max(window, 1));
  if (c.invalid.empty() && c.unsupported.empty()) {
    const size_t need = ml4_workspace_bytes(ML4_ENTRY_MLA, s, n_heads, window);
    c.ws(ws_bytes < need, bytes_msg("window-MLA workspace", need, ws_bytes));
    c.ws(need && (!ws || !aligned(ws, 256)), "workspace must be non-NULL and 256-byte aligned");
  }
  if (int rc = c.finish("ml4_window_mla_decode")) return rc;
  ml4::MlaLaunch a{};
  a.s = view(s);
  a.pool = kv->pool;
  a.num_blocks = kv->num_blocks;
  a.fp8 = true;
  a.bf16_rows = kv->format == ML4_LAT_BF16_1152;
  a.window = window;
  a.q = q;
  a.n_heads = n_heads;
  a.rope_dim = rope_dim;
  a.top_k = window;
  a.softmax_scale = softmax_scale;
  a.ssmax_s = ssmax_s;
  a.out = out;
  a.lse = lse;
  a.ws = ws;
  a.fault = fault;
  return launch_status(ml4::launch_mla(a, stream), "ml4_window_mla_decode");
}

}  // extern "C"

namespace {

// The fused layer.  static_scratch: the no-allocation form -- instead of the caller's
// workspace, the library's fixed scratch array (its size checked here, its device address
// looked up only after every check has passed).
int fused_layer(const char* entry, const ml4_layer* layers, int32_t layer, const ml4_seqs* s,
                const ml4_cache* lat_caches, const ml4_cache* idx_caches, int32_t n_layers,
                const void* q_idx, int32_t q_idx_dtype, const float* q_idx_scale,
                const float* w_idx, const void* q_mla, int32_t q_mla_dtype,
                int32_t* const* topk_bufs, int32_t* const* topk_lens, void* out,
                int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, bool static_scratch,
                uint32_t* fault, hipStream_t stream) {
  Checks c;
  check_seqs(c, s);
  c.bad(layers == nullptr, "layers is NULL");
  c.bad(n_layers < 1, "n_layers must be >= 1");
  c.bad(!lat_caches || !topk_bufs || !topk_lens, "lat_caches, topk_bufs, topk_lens must be non-NULL");
  c.bad(layer < 0 || layer >= n_layers, "layer outside 0 .. n_layers-1");
  if (!layers || n_layers < 1 || !lat_caches || !topk_bufs || !topk_lens || layer < 0 ||
      layer >= n_layers)
    return c.finish(entry);
  const ml4_layer* L = &layers[layer];
  const int l = layer;
  c.bad(L->layer != l, "layers[layer].layer differs from layer");
  const int tgt = L->kv_sharing_target_layer, src = L->topk_source_layer;
  const bool tgt_ok = tgt == -1 || (tgt >= 0 && tgt < l);
  const bool src_ok = src == -1 || (src >= 0 && src < l);
  c.bad(!tgt_ok, "kv_sharing_target_layer must be -1 or an earlier layer");
  c.bad(!src_ok, "topk_source_layer must be -1 or an earlier layer");
  if (!tgt_ok || !src_ok) return c.finish(entry);
  // [blog, 跨层 KV 共享]: a consumer reads the cache of a layer that owns one (no chains);
  // [blog, Model architecture]: a shared-indexer layer reuses the top-k of a layer that runs
  // its own indexer, with the same top_k (the row stride of that layer's top-k buffer).
  if (tgt >= 0) {
    c.bad(layers[tgt].layer != tgt, "layers[kv_sharing_target_layer].layer differs from its index");
    c.bad(layers[tgt].kv_sharing_target_layer != -1,
          "kv_sharing_target_layer names a consumer layer: the target must own its cache");
  }
  if (src >= 0) {
    c.bad(layers[src].layer != src, "layers[topk_source_layer].layer differs from its index");
    c.bad(layers[src].topk_source_layer != -1,
          "topk_source_layer names a shared-indexer layer: the source must run its own indexer");
    c.bad(layers[src].top_k != L->top_k,
          "top_k differs from the topk_source_layer's top_k (the shared top-k rows' stride)");
  }
  const int lat_layer = tgt >= 0 ? tgt : l;
  const bool own_indexer = src < 0;
  const int topk_layer = own_indexer ? l : src;
  c.bad(!topk_bufs[topk_layer] || !topk_lens[topk_layer],
        own_indexer ? "topk_bufs[layer] / topk_lens[layer] must be non-NULL"
                    : "topk_bufs[topk_source_layer] / topk_lens[topk_source_layer] must be non-NULL");
  const int64_t ld = s ? (int64_t)ml4::align_up((size_t)s->max_seq_len, 4) : 0;
  if (own_indexer) {
    c.bad(!idx_caches, "idx_caches is NULL for an indexer layer");
    if (idx_caches)
      check_indexer(c, &idx_caches[l], q_idx, q_idx_dtype, w_idx, L->idx_heads, L->idx_ssmax_s);
    check_topk(c, L->top_k, topk_bufs[topk_layer], topk_lens[topk_layer]);
  }
  check_mla(c, &lat_caches[lat_layer], q_mla, q_mla_dtype, L->mla_heads, L->rope_dim,
            topk_bufs[topk_layer], topk_lens[topk_layer], L->top_k, L->softmax_scale, L->ssmax_s,
            out, out_dtype);
  c.unsup(lat_caches[lat_layer].format == ML4_LAT_E4M3_576,
          "the fused layer takes ML4_LAT_FP8_656, ML4_LAT_BF16_1152 or ML4_LAT_F32 latent "
          "caches (ML4_LAT_E4M3_576: ml4_sparse_mla_decode_e4m3)");
  if (c.invalid.empty() && c.unsupported.empty() && s) {
    const size_t need = ml4_workspace_bytes(ML4_ENTRY_LAYER, s, L->mla_heads, L->top_k);
    if (static_scratch) {
      c.unsupported.push_back(need > (size_t)ML4_STATIC_SCRATCH_BYTES
                                  ? bytes_msg("this batch's scratch (above the fixed "
                                              "ML4_STATIC_SCRATCH_BYTES; use "
                                              "ml4_sparse_attn_layer with a workspace)",
                                              need, (size_t)ML4_STATIC_SCRATCH_BYTES)
                                  : std::string());
      if (c.unsupported.back().empty()) c.unsupported.pop_back();
    } else {
      c.ws(ws_bytes < need, bytes_msg("layer workspace", need, ws_bytes));
      c.ws(!ws || !aligned(ws, 256), "workspace must be non-NULL and 256-byte aligned");
    }
  }
  if (int rc = c.finish(entry)) return rc;
  if (static_scratch) {
    const hipError_t e = ml4::static_scratch_address(&ws);
    if (e != hipSuccess) return launch_status(e, entry);
    ws_bytes = ML4_STATIC_SCRATCH_BYTES;
  }
  float* scores = static_cast<float*>(ws);

  const ml4::SeqView v = view(s);
  char* wsp = static_cast<char*>(ws);
  const size_t sc_bytes = layer_scores_bytes(s);
  const size_t tk_bytes = ml4::align_up(ml4::topk_ws_bytes(v, L->top_k), 256);
  hipError_t e = hipSuccess;
  if (own_indexer) {
    ml4::IndexerLaunch ia{};
    ia.s = v;
    ia.pool = idx_caches[l].pool;
    ia.num_blocks = idx_caches[l].num_blocks;
    ia.fp8 = idx_caches[l].format == ML4_IDX_FP8_132;
    ia.q = q_idx;
    ia.q_scale = q_idx_scale;
    ia.w = w_idx;
    ia.n_heads = L->idx_heads;
    ia.ssmax_s = L->idx_ssmax_s;
    ia.scores = scores;
    ia.ld = ld;
    ia.fault = fault;
    e = ml4::launch_indexer(ia, stream);
    if (e != hipSuccess) return launch_status(e, entry);
    ml4::TopkLaunch ta{};
    ta.s = v;
    ta.scores = scores;
    ta.ld = ld;
    ta.top_k = L->top_k;
    ta.idx = topk_bufs[l];
    ta.len = topk_lens[l];
    ta.ws = wsp + sc_bytes;
    ta.fault = fault;
    e = ml4::launch_topk(ta, stream);
    if (e != hipSuccess) return launch_status(e, entry);
  }
  ml4::MlaLaunch ma{};
  ma.s = v;
  ma.pool = lat_caches[lat_layer].pool;
  ma.num_blocks = lat_caches[lat_layer].num_blocks;
  ma.fp8 = lat_caches[lat_layer].format != ML4_LAT_F32;
  ma.bf16_rows = lat_caches[lat_layer].format == ML4_LAT_BF16_1152;
  ma.q = q_mla;
  ma.n_heads = L->mla_heads;
  ma.rope_dim = L->rope_dim;
  ma.idx = topk_bufs[topk_layer];
  ma.len = topk_lens[topk_layer];
  ma.top_k = L->top_k;
  ma.softmax_scale = L->softmax_scale;
  ma.ssmax_s = L->ssmax_s;
  ma.out = out;
  ma.lse = lse;
  ma.ws = wsp + sc_bytes + tk_bytes;
  ma.fault = fault;
  return launch_status(ml4::launch_mla(ma, stream), entry);
}

}  // namespace

extern "C" {

int ml4_sparse_attn_layer(const ml4_layer* layers, int32_t layer, const ml4_seqs* s,
                          const ml4_cache* lat_caches, const ml4_cache* idx_caches,
                          int32_t n_layers, const void* q_idx, int32_t q_idx_dtype,
                          const float* q_idx_scale, const float* w_idx, const void* q_mla,
                          int32_t q_mla_dtype, int32_t* const* topk_bufs,
                          int32_t* const* topk_lens, void* out, int32_t out_dtype, float* lse,
                          void* ws, size_t ws_bytes, uint32_t* fault, hipStream_t stream) {
  return fused_layer("ml4_sparse_attn_layer", layers, layer, s, lat_caches, idx_caches,
                     n_layers, q_idx, q_idx_dtype, q_idx_scale, w_idx, q_mla, q_mla_dtype,
                     topk_bufs, topk_lens, out, out_dtype, lse, ws, ws_bytes, false, fault,
                     stream);
}

int ml4_sparse_attn_layer_static(const ml4_layer* layers, int32_t layer, const ml4_seqs* s,
                                 const ml4_cache* lat_caches, const ml4_cache* idx_caches,
                                 int32_t n_layers, const void* q_idx, int32_t q_idx_dtype,
                                 const float* q_idx_scale, const float* w_idx,
                                 const void* q_mla, int32_t q_mla_dtype,
                                 int32_t* const* topk_bufs, int32_t* const* topk_lens,
                                 void* out, int32_t out_dtype, float* lse, uint32_t* fault,
                                 hipStream_t stream) {
  return fused_layer("ml4_sparse_attn_layer_static", layers, layer, s, lat_caches, idx_caches,
                     n_layers, q_idx, q_idx_dtype, q_idx_scale, w_idx, q_mla, q_mla_dtype,
                     topk_bufs, topk_lens, out, out_dtype, lse, nullptr, 0, true, fault, stream);
}

namespace {

// e4m3: the ml4_latent_cache_write_e4m3 entry (kv_scale used); else kv_scale is ignored.
int cache_write(const char* entry, bool latent, bool e4m3, const ml4_cache* cache,
                int32_t block_size, const void* src, int32_t src_dtype, const void* rope,
                int32_t rope_dim, float kv_scale, int64_t n_tokens,
                const int64_t* slot_mapping, uint32_t* fault, hipStream_t stream) {
  Checks c;
  if (!cache) {
    c.bad(true, latent ? "lat_cache is NULL" : "idx_cache is NULL");
  } else {
    c.bad(!cache->pool, "cache.pool is NULL");
    c.bad(!aligned(cache->pool, 16), "cache.pool must be 16-byte aligned");
    c.bad(cache->num_blocks < 1, "cache.num_blocks must be >= 1");
    if (e4m3) {
      c.unsup(cache->format != ML4_LAT_E4M3_576, "cache.format must be ML4_LAT_E4M3_576");
    } else if (latent) {
      c.unsup(cache->format == ML4_LAT_E4M3_576,
              "an ML4_LAT_E4M3_576 cache takes a scale: use ml4_latent_cache_write_e4m3");
      c.unsup(cache->format != ML4_LAT_FP8_656 && cache->format != ML4_LAT_BF16_1152 &&
                  cache->format != ML4_LAT_E4M3_576,
              "cache.format must be ML4_LAT_FP8_656 or ML4_LAT_BF16_1152");
    } else
      c.unsup(cache->format != ML4_IDX_FP8_132, "cache.format must be ML4_IDX_FP8_132");
  }
  c.bad(!pow2(block_size), "block_size must be a power of two");
  c.unsup(pow2(block_size) && (block_size < 16 || block_size > 65536),
          "block_size outside 16 .. 65536");
  c.bad(n_tokens < 0, "n_tokens must be >= 0");
  c.unsup(src_dtype != ML4_BF16 && src_dtype != ML4_F32, "src_dtype must be ML4_BF16 or ML4_F32");
  if (n_tokens > 0) {
    c.bad(!src, "source values are NULL");
    c.bad(!slot_mapping, "slot_mapping is NULL");
    c.bad(!aligned(src, 16), "source values must be 16-byte aligned");
    c.bad(!aligned(slot_mapping, 8), "slot_mapping must be 8-byte aligned");
  }
  if (latent) {
    c.unsup(rope_dim != 0 && rope_dim != ML4_ROPE_DIM, "rope_dim must be 0 or 64");
    c.bad(rope_dim && n_tokens > 0 && (!rope || !aligned(rope, 8)),
          "k_rope must be non-NULL and 8-byte aligned when rope_dim is 64");
  }
  if (e4m3)
    c.bad(!(std::isfinite(kv_scale) && kv_scale > 0.f), "kv_scale must be finite and > 0");
  c.unsup(n_tokens > ((int64_t)1 << 31), "n_tokens above 2^31");
  if (int rc = c.finish(entry)) return rc;
  ml4::CacheWriteLaunch a{};
  a.latent = latent;
  a.bf16_rows = latent && cache->format == ML4_LAT_BF16_1152;
  a.e4m3_rows = e4m3;
  a.kv_scale = kv_scale;
  a.pool = const_cast<void*>(cache->pool);   // the write entries own the rows they write
  a.capacity = cache->num_blocks * (int64_t)block_size;
  a.src = src;
  a.bf16 = src_dtype == ML4_BF16;
  a.rope = rope_dim ? rope : nullptr;
  a.rope_dim = rope_dim;
  a.n_tokens = n_tokens;
  a.slot_mapping = slot_mapping;
  a.fault = fault;
  return launch_status(ml4::launch_cache_write(a, stream), entry);
}

}  // namespace

int ml4_index_cache_write(const ml4_cache* idx_cache, int32_t block_size, const void* k,
                          int32_t src_dtype, int64_t n_tokens, const int64_t* slot_mapping,
                          uint32_t* fault, hipStream_t stream) {
  return cache_write("ml4_index_cache_write", false, false, idx_cache, block_size, k,
                     src_dtype, nullptr, 0, 0.f, n_tokens, slot_mapping, fault, stream);
}

int ml4_latent_cache_write(const ml4_cache* lat_cache, int32_t block_size, const void* c,
                           int32_t src_dtype, const void* k_rope, int32_t rope_dim,
                           int64_t n_tokens, const int64_t* slot_mapping, uint32_t* fault,
                           hipStream_t stream) {
  return cache_write("ml4_latent_cache_write", true, false, lat_cache, block_size, c,
                     src_dtype, k_rope, rope_dim, 0.f, n_tokens, slot_mapping, fault, stream);
}

int ml4_latent_cache_write_e4m3(const ml4_cache* lat_cache, int32_t block_size, const void* c,
                                int32_t src_dtype, const void* k_rope, int32_t rope_dim,
                                float kv_scale, int64_t n_tokens, const int64_t* slot_mapping,
                                uint32_t* fault, hipStream_t stream) {
  return cache_write("ml4_latent_cache_write_e4m3", true, true, lat_cache, block_size, c,
                     src_dtype, k_rope, rope_dim, kv_scale, n_tokens, slot_mapping, fault,
                     stream);
}

int ml4_topk_merge(int32_t rows, int32_t n_shards, const float* cand_scores,
                   const int32_t* cand_pos, const int32_t* cand_len, int64_t ld_cand,
                   int32_t top_k, int32_t* topk_idx, int32_t* topk_len, uint32_t* fault,
                   hipStream_t stream) {
  Checks c;
  c.bad(rows < 0, "rows must be >= 0");
  c.bad(n_shards < 1, "n_shards must be >= 1");
  c.bad(ld_cand < 1, "ld_cand must be >= 1");
  c.unsup(n_shards >= 1 && ld_cand >= 1 && (int64_t)n_shards * ld_cand > 16384,
          "n_shards * ld_cand above 16384");
  c.bad(top_k < 1 || top_k > ML4_MAX_TOPK, "top_k must be in 1 .. 2048");
  if (rows > 0) {
    c.bad(!cand_scores || !cand_pos || !cand_len, "candidate arrays must be non-NULL");
    c.bad(!topk_idx || !topk_len, "topk_idx and topk_len must be non-NULL");
    c.bad(!aligned(cand_scores, 4) || !aligned(cand_pos, 4) || !aligned(cand_len, 4) ||
              !aligned(topk_idx, 4) || !aligned(topk_len, 4),
          "arrays must be 4-byte aligned");
  }
  if (int rc = c.finish("ml4_topk_merge")) return rc;
  ml4::MergeLaunch a{};
  a.rows = rows;
  a.n_shards = n_shards;
  a.ld = ld_cand;
  a.cand_scores = cand_scores;
  a.cand_pos = cand_pos;
  a.cand_len = cand_len;
  a.top_k = top_k;
  a.idx = topk_idx;
  a.len = topk_len;
  a.fault = fault;
  return launch_status(ml4::launch_topk_merge(a, stream), "ml4_topk_merge");
}

int ml4_lse_combine(int32_t rows, int32_t n_heads, int32_t n_shards, int32_t head_dim,
                    const float* o_parts, const float* lse_parts, void* out, int32_t out_dtype,
                    float* lse, hipStream_t stream) {
  Checks c;
  c.bad(rows < 0, "rows must be >= 0");
  c.bad(n_heads < 1 || n_heads > 65535, "n_heads must be in 1 .. 65535");
  c.bad(n_shards < 1, "n_shards must be >= 1");
  c.bad(head_dim < 1 || head_dim > 4096, "head_dim must be in 1 .. 4096");
  c.unsup(out_dtype != ML4_BF16 && out_dtype != ML4_F32, "out_dtype must be ML4_BF16 or ML4_F32");
  if (rows > 0) {
    c.bad(!o_parts || !lse_parts || !out, "o_parts, lse_parts and out must be non-NULL");
    c.bad(!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(lse, 4) ||
              !aligned(out, out_dtype == ML4_F32 ? 4 : 2),
          "arrays misaligned");
  }
  if (int rc = c.finish("ml4_lse_combine")) return rc;
  ml4::LseCombineLaunch a{};
  a.rows = rows;
  a.n_heads = n_heads;
  a.n_shards = n_shards;
  a.head_dim = head_dim;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.out = out;
  a.out_bf16 = out_dtype == ML4_BF16;
  a.lse = lse;
  return launch_status(ml4::launch_lse_combine(a, stream), "ml4_lse_combine");
}

int ml4_fault_query(const uint32_t* fault, uint32_t* bits, hipStream_t stream) {
  if (!fault || !bits) {
    g_last_error = "ml4_fault_query: invalid: fault and bits must be non-NULL\n";
    return ML4_E_INVALID;
  }
  uint32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, fault, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return launch_status(e, "ml4_fault_query");
  *bits = h;
  return h ? ML4_E_DEVICE_FAULT : ML4_OK;
}

}  // extern "C"
