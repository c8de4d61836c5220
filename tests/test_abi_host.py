"""Host-side tests of the C ABI: the library loads, exports every symbol the header
declares, and its default-deny validation rejects bad calls -- listing every failed check
-- without touching a GPU (nothing is launched when a check fails)."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ml4dsa.h")

M = pytest.importorskip("sparse_attention_decode_dsa_amd.ml4dsa",
                        reason="libml4dsa.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ml4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_bound_entry_points():
    assert header_functions() == sorted(M.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(M.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_header_constants_match_binding_and_pages():
    text = open(HEADER).read()
    def define(n):
        return int(re.search(rf"#define {n} (\d+)", text).group(1))
    assert define("ML4_IDX_ROW_FP8") == 132 and define("ML4_LAT_ROW_FP8") == 656
    assert define("ML4_KV_LORA") == 512 and define("ML4_ROPE_DIM") == 64
    assert define("ML4_MAX_TOPK") == 2048 and define("ML4_ABI_VERSION") == M.ML4_ABI_VERSION
    assert M.ml4_abi_version() == M.ML4_ABI_VERSION
    bits = {m.group(1): 1 << int(m.group(2))
            for m in re.finditer(r"(ML4_FAULT_\w+) = 1u << (\d+)", text)}
    assert bits and all(getattr(M, k) == v for k, v in bits.items())


def _seqs(**kw):
    s = M.ml4_seqs()
    s.batch, s.total_q, s.max_seq_len, s.max_q_per_seq = 1, 1, 4096, 1
    s.block_size, s.max_blocks_per_seq = 64, 64
    s.seq_lens = s.q_start = s.q_pos = s.block_table = 0x1000
    for k, v in kw.items():
        setattr(s, k, v)
    return s


def _cache(fmt, pool=0x10000):
    c = M.ml4_cache()
    c.pool, c.num_blocks, c.format = pool, 64, fmt
    return c


def test_indexer_default_deny_lists_every_reason():
    s = _seqs(block_size=48, seq_lens=0)
    rc = M.ml4_indexer_score(s, _cache(M.ML4_IDX_FP8_132, pool=0x10004), 0x2000, M.ML4_F32,
                             None, None, 24, 0.0, 0x3000, 102, stream=0, check=False)
    assert rc == M.ML4_E_INVALID
    msg = M.ml4_last_error()
    for needle in ["block_size must be a power of two", "seqs arrays", "16-byte aligned",
                   "needs ML4_FP8_E4M3 queries", "w is NULL", "ld_scores < max_seq_len",
                   "ld_scores must be a multiple of 4", "n_heads must be a multiple of 16"]:
        assert needle in msg, (needle, msg)
    assert len(msg.strip().splitlines()) >= 8


def test_unsupported_and_workspace_codes():
    s = _seqs()
    rc = M.ml4_topk_select(s, 0x4000, 4096, 4096, 0x5000, 0x6000, stream=0, check=False)
    assert rc == M.ML4_E_UNSUPPORTED and "top_k above 2048" in M.ml4_last_error()
    big = _seqs(max_seq_len=1 << 20, max_blocks_per_seq=(1 << 20) // 64)
    need = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, big, 0, 2048)
    assert need > 0
    rc = M.ml4_topk_select(big, 0x4000, 1 << 20, 2048, 0x5000, 0x6000, None, 0, stream=0,
                           check=False)
    assert rc == M.ML4_E_WORKSPACE and "workspace" in M.ml4_last_error()


def test_mla_default_deny():
    s = _seqs()
    rc = M.ml4_sparse_mla_decode(s, _cache(M.ML4_LAT_FP8_656), 0x7000, M.ML4_F32, 20, 32,
                                 0x5000, None, 4096, -1.0, float("nan"), 0x8000, M.ML4_F32,
                                 stream=0, check=False)
    assert rc == M.ML4_E_INVALID
    msg = M.ml4_last_error()
    for needle in ["needs ML4_BF16 queries", "writes ML4_BF16 outputs",
                   "n_heads must be a multiple of 16", "rope_dim must be 64 or 0",
                   "topk_idx and topk_len", "top_k above 2048", "softmax_scale",
                   "ssmax_s must be finite"]:
        assert needle in msg, (needle, msg)


def test_e4m3_mla_default_deny():
    """The plain-E4M3 layout carries scales: the generic entry refuses it, and its own entry
    checks the format, both scales, the output dtype and the shared MLA arguments."""
    s = _seqs()
    rc = M.ml4_sparse_mla_decode(s, _cache(M.ML4_LAT_E4M3_576), 0x7000, M.ML4_FP8_E4M3, 16,
                                 64, 0x5000, 0x5100, 2048, 0.04, 0.0, 0x8000, M.ML4_BF16,
                                 stream=0, check=False)
    assert rc == M.ML4_E_INVALID and "use ml4_sparse_mla_decode_e4m3" in M.ml4_last_error()
    rc = M.ml4_sparse_mla_decode_e4m3(s, _cache(M.ML4_LAT_FP8_656), float("inf"), 0x7008, None,
                                      24, 64, 0x5000, 0x5100, 2048, 0.04, 0.0, 0x8000,
                                      M.ML4_F32, stream=0, check=False)
    assert rc == M.ML4_E_INVALID
    msg = M.ml4_last_error()
    for needle in ["kv.format must be ML4_LAT_E4M3_576", "kv_scale must be finite and > 0",
                   "q_scale is NULL", "q must be 16-byte aligned",
                   "n_heads must be a multiple of 16"]:
        assert needle in msg, (needle, msg)
    rc = M.ml4_sparse_mla_decode_e4m3(s, _cache(M.ML4_LAT_E4M3_576), 0.01, 0x7000, 0x7100,
                                      16, 64, 0x5000, 0x5100, 2048, 0.04, 0.0, 0x8000,
                                      M.ML4_F32, stream=0, check=False)
    assert rc == M.ML4_E_INVALID
    assert "ML4_FP8_E4M3 queries and ML4_BF16 outputs" in M.ml4_last_error()
    # window attention and the fused layer take the other layouts only
    rc = M.ml4_window_mla_decode(s, _cache(M.ML4_LAT_E4M3_576), 0x7000, M.ML4_FP8_E4M3, 16,
                                 64, 2048, 0.04, 0.0, 0x8000, M.ML4_BF16, stream=0,
                                 check=False)
    assert rc == M.ML4_E_UNSUPPORTED and "window attention" in M.ml4_last_error()
    L = M.ml4_layer()
    L.layer, L.kv_sharing_target_layer, L.topk_source_layer = 0, -1, -1
    L.rope_dim, L.top_k, L.idx_heads, L.mla_heads = 64, 2048, 64, 128
    L.softmax_scale = 0.04
    rc = M.ml4_sparse_attn_layer([L], 0, s, [_cache(M.ML4_LAT_E4M3_576)],
                                 [_cache(M.ML4_IDX_FP8_132)], 0x100, M.ML4_FP8_E4M3, None,
                                 0x100, 0x100, M.ML4_FP8_E4M3, [0x100], [0x100], 0x100,
                                 M.ML4_BF16, stream=0, check=False)
    assert rc in (M.ML4_E_UNSUPPORTED, M.ML4_E_INVALID)
    assert "ml4_sparse_mla_decode_e4m3" in M.ml4_last_error()


def _layer(l, tgt=-1, src=-1, top_k=2048):
    L = M.ml4_layer()
    L.layer, L.kv_sharing_target_layer, L.topk_source_layer = l, tgt, src
    L.rope_dim, L.top_k, L.idx_heads, L.mla_heads = 64, top_k, 64, 128
    L.softmax_scale = 0.04
    return L


def _fused(layers, l, ws_bytes=0):
    n = len(layers)
    return M.ml4_sparse_attn_layer(layers, l, _seqs(), [_cache(M.ML4_LAT_FP8_656)] * n,
                                   [_cache(M.ML4_IDX_FP8_132)] * n, 0x100, M.ML4_FP8_E4M3, None,
                                   0x100, 0x100, M.ML4_BF16, [0x100] * n, [0x100] * n, 0x100,
                                   M.ML4_BF16, stream=0, check=False, ws_bytes=ws_bytes)


def test_layer_modes_are_validated():
    rc = _fused([_layer(0), _layer(1, tgt=1, src=2), _layer(2)], 1)
    assert rc == M.ML4_E_INVALID
    msg = M.ml4_last_error()
    assert "kv_sharing_target_layer must be -1 or an earlier layer" in msg
    assert "topk_source_layer must be -1 or an earlier layer" in msg
    rc = _fused([_layer(0), _layer(5)], 1)
    assert rc == M.ML4_E_INVALID and "layers[layer].layer differs" in M.ml4_last_error()


def test_layer_roles_no_chains_and_indexer_owner_sources():
    """[blog, 跨层 KV 共享]: a consumer reads a layer that owns its cache, never another
    consumer; a shared-indexer layer reuses the top-k of a layer that runs its own indexer,
    with the same top_k (the shared rows' stride).  Each violation is listed; a valid
    three-layer chain (owner, shared-indexer, consumer) passes validation up to the
    workspace check (no workspace given, nothing launched)."""
    layers = [_layer(0), _layer(1, tgt=0), _layer(2, tgt=1)]          # consumer of a consumer
    assert _fused(layers, 2) == M.ML4_E_INVALID
    assert "the target must own its cache" in M.ml4_last_error()
    layers = [_layer(0), _layer(1, src=0), _layer(2, src=1)]          # sharer of a sharer
    assert _fused(layers, 2) == M.ML4_E_INVALID
    assert "the source must run its own indexer" in M.ml4_last_error()
    layers = [_layer(0, top_k=1024), _layer(1, src=0, top_k=2048)]    # stride mismatch
    assert _fused(layers, 1) == M.ML4_E_INVALID
    assert "top_k differs from the topk_source_layer's top_k" in M.ml4_last_error()
    layers = [_layer(0), _layer(1, tgt=0, src=0), _layer(2, tgt=1, src=1)]   # both at once
    assert _fused(layers, 2) == M.ML4_E_INVALID
    msg = M.ml4_last_error()
    assert "the target must own its cache" in msg and "the source must run its own indexer" in msg
    layers = [_layer(0), _layer(1, src=0), _layer(2, tgt=0)]          # the 1M-key three layers
    for l in range(3):
        assert _fused(layers, l) == M.ML4_E_WORKSPACE, M.ml4_last_error()


def test_static_scratch_entry_validates_and_refuses_oversized_batches():
    """The no-allocation fused entry runs the same default-deny checks (nothing launched, no
    device touched when a check fails) and refuses a batch whose scratch exceeds the fixed
    array, naming both sizes."""
    text = open(HEADER).read()
    assert re.search(r"#define ML4_STATIC_SCRATCH_BYTES \(64u << 20\)", text)
    assert M.ML4_STATIC_SCRATCH_BYTES == 64 << 20
    layers = [_layer(0)]
    args = ([_cache(M.ML4_LAT_FP8_656)], [_cache(M.ML4_IDX_FP8_132)], 0x100, M.ML4_FP8_E4M3,
            None, 0x100, 0x100, M.ML4_BF16, [0x100], [0x100], 0x100, M.ML4_BF16)
    big = _seqs(total_q=512, max_q_per_seq=512, max_seq_len=65536, max_blocks_per_seq=1024)
    rc = M.ml4_sparse_attn_layer_static(layers, 0, big, *args, stream=0, check=False)
    msg = M.ml4_last_error()
    assert rc == M.ML4_E_UNSUPPORTED and "ML4_STATIC_SCRATCH_BYTES" in msg
    assert str(M.ml4_workspace_bytes(M.ML4_ENTRY_LAYER, big, 128, 2048)) in msg
    assert str(64 << 20) in msg
    bad = [_layer(0), _layer(1, tgt=0), _layer(2, tgt=1)]
    rc = M.ml4_sparse_attn_layer_static(bad, 2, _seqs(block_size=48),
                                        [_cache(M.ML4_LAT_FP8_656)] * 3,
                                        [_cache(M.ML4_IDX_FP8_132)] * 3, 0x100, M.ML4_FP8_E4M3,
                                        None, 0x100, 0x100, M.ML4_BF16, [0x100] * 3,
                                        [0x100] * 3, 0x100, M.ML4_BF16, stream=0, check=False)
    msg = M.ml4_last_error()
    assert rc == M.ML4_E_INVALID
    assert "the target must own its cache" in msg and "block_size must be a power of two" in msg
    assert msg.startswith("ml4_sparse_attn_layer_static:")


def test_fault_query_rejects_null():
    rc = M.LIB.ml4_fault_query(None, None, None)
    assert rc == M.ML4_E_INVALID


def test_cache_write_default_deny_lists_every_reason():
    """Host validation of the cache-write entries: every failed check listed, nothing
    launched; zero tokens is a valid no-op."""
    c = M.ml4_cache()
    c.pool, c.num_blocks, c.format = 0, 0, M.ML4_IDX_F32      # fp32 rows are read-only
    rc = M.ml4_index_cache_write(c, 48, None, 7, 5, None, None, stream=0, check=False)
    msg = M.ml4_last_error()
    assert rc == M.ML4_E_INVALID
    for frag in ("cache.pool is NULL", "num_blocks", "block_size", "src_dtype",
                 "source values are NULL", "slot_mapping is NULL", "ML4_IDX_FP8_132"):
        assert frag in msg, (frag, msg)
    c2 = M.ml4_cache()
    c2.pool, c2.num_blocks, c2.format = 4096, 4, M.ML4_LAT_FP8_656
    rc = M.ml4_latent_cache_write(c2, 64, None, M.ML4_BF16, None, 32, 0, None, None, stream=0,
                                  check=False)
    assert rc == M.ML4_E_UNSUPPORTED and "rope_dim" in M.ml4_last_error()
    rc = M.ml4_latent_cache_write(c2, 64, None, M.ML4_BF16, None, 64, 0, None, None, stream=0,
                                  check=False)
    assert rc == M.ML4_OK
    # source rows are read as 16-byte vectors: an address off a 16-byte boundary is refused
    # (host validation only: nothing is launched, the pointers are never dereferenced)
    rc = M.ml4_index_cache_write(c2, 64, 4096 + 8, M.ML4_BF16, 5, 8192, None, stream=0,
                                 check=False)
    assert rc == M.ML4_E_INVALID and "16-byte aligned" in M.ml4_last_error()


def test_second_layout_cache_writes_default_deny():
    """The plain-E4M3 latent cache is written only through the entry that takes its scale;
    that entry refuses any other format and a scale that is not finite and positive; the
    bf16 cache goes through the generic entry."""
    c = M.ml4_cache()
    c.pool, c.num_blocks, c.format = 4096, 4, M.ML4_LAT_E4M3_576
    rc = M.ml4_latent_cache_write(c, 64, None, M.ML4_BF16, None, 0, 0, None, None, stream=0,
                                  check=False)
    assert rc == M.ML4_E_UNSUPPORTED and "ml4_latent_cache_write_e4m3" in M.ml4_last_error()
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        rc = M.ml4_latent_cache_write_e4m3(c, 64, None, M.ML4_BF16, None, 0, bad, 0, None,
                                           None, stream=0, check=False)
        assert rc == M.ML4_E_INVALID and "kv_scale" in M.ml4_last_error(), bad
    assert M.ml4_latent_cache_write_e4m3(c, 64, None, M.ML4_BF16, None, 64, 0.5, 0, None,
                                         None, stream=0, check=False) == M.ML4_OK
    c.format = M.ML4_LAT_FP8_656
    rc = M.ml4_latent_cache_write_e4m3(c, 64, None, M.ML4_BF16, None, 0, 0.5, 0, None, None,
                                       stream=0, check=False)
    assert rc == M.ML4_E_UNSUPPORTED and "ML4_LAT_E4M3_576" in M.ml4_last_error()
    c.format = M.ML4_LAT_BF16_1152
    assert M.ml4_latent_cache_write(c, 64, None, M.ML4_F32, None, 64, 0, None, None,
                                    stream=0, check=False) == M.ML4_OK
    c.format = M.ML4_LAT_F32
    rc = M.ml4_latent_cache_write(c, 64, None, M.ML4_F32, None, 64, 0, None, None, stream=0,
                                  check=False)
    assert rc == M.ML4_E_UNSUPPORTED
