"""ctypes binding of libml4dsa.so: the C entry points under the same names.

Argument marshalling only: every step runs in the HIP library.  torch supplies device
memory and streams.  There is no fallback: if the library is not built this module fails
to load, loudly.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libml4dsa.so")

# ---- constants mirrored from include/ml4dsa.h
ML4_ABI_VERSION = 6
ML4_OK, ML4_E_INVALID, ML4_E_UNSUPPORTED, ML4_E_WORKSPACE, ML4_E_LAUNCH, ML4_E_DEVICE_FAULT = (
    0, -1, -2, -3, -4, -5)
ML4_F32, ML4_BF16, ML4_FP8_E4M3 = 0, 1, 2
ML4_IDX_F32, ML4_IDX_FP8_132 = 0, 1
ML4_LAT_F32, ML4_LAT_FP8_656, ML4_LAT_BF16_1152, ML4_LAT_E4M3_576 = 0, 1, 2, 3
ML4_FAULT_BLOCK_ID, ML4_FAULT_TOPK_INDEX, ML4_FAULT_NAN_SCORE, ML4_FAULT_QPOS = 1, 2, 4, 8
ML4_FAULT_RANGE = 16
ML4_ENTRY_TOPK, ML4_ENTRY_MLA, ML4_ENTRY_LAYER = 1, 2, 3
ML4_STATIC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("ml4_indexer_score", "ml4_topk_select", "ml4_sparse_mla_decode",
           "ml4_sparse_mla_decode_e4m3", "ml4_sparse_attn_layer", "ml4_sparse_attn_layer_static",
           "ml4_window_mla_decode",
           "ml4_index_cache_write", "ml4_latent_cache_write", "ml4_latent_cache_write_e4m3",
           "ml4_topk_merge", "ml4_lse_combine", "ml4_workspace_bytes", "ml4_last_error",
           "ml4_fault_query", "ml4_abi_version", "ml4_probe_read", "ml4_probe_mfma")


class ml4_seqs(C.Structure):
    _fields_ = [("batch", C.c_int32), ("total_q", C.c_int32), ("max_seq_len", C.c_int32),
                ("max_q_per_seq", C.c_int32), ("block_size", C.c_int32),
                ("max_blocks_per_seq", C.c_int32), ("seq_lens", C.c_void_p),
                ("q_start", C.c_void_p), ("q_pos", C.c_void_p), ("block_table", C.c_void_p)]


class ml4_cache(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("num_blocks", C.c_int64), ("format", C.c_int32)]


class ml4_layer(C.Structure):
    _fields_ = [("layer", C.c_int32), ("kv_sharing_target_layer", C.c_int32),
                ("topk_source_layer", C.c_int32), ("rope_dim", C.c_int32),
                ("top_k", C.c_int32), ("idx_heads", C.c_int32), ("mla_heads", C.c_int32),
                ("softmax_scale", C.c_float), ("ssmax_s", C.c_float),
                ("idx_ssmax_s", C.c_float)]


class ML4Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"ml4 status {code}: {message.strip()}")
        self.code = code
        self.message = message


def _load() -> C.CDLL:
    # torch ships its own HIP runtime; importing it first makes libml4dsa.so bind to that
    # same runtime instead of loading a second one into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build the HIP library first "
                          "(python -m sparse_attention_decode_dsa_amd.build)")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    P = C.POINTER
    lib.ml4_abi_version.restype = C.c_int
    lib.ml4_abi_version.argtypes = []
    lib.ml4_last_error.restype = C.c_char_p
    lib.ml4_last_error.argtypes = []
    lib.ml4_workspace_bytes.restype = sz
    lib.ml4_workspace_bytes.argtypes = [i32, P(ml4_seqs), i32, i32]
    lib.ml4_fault_query.restype = C.c_int
    lib.ml4_fault_query.argtypes = [vp, P(C.c_uint32), vp]
    lib.ml4_indexer_score.restype = C.c_int
    lib.ml4_indexer_score.argtypes = [P(ml4_seqs), P(ml4_cache), vp, i32, vp, vp, i32, f32, vp,
                                      i64, vp, vp]
    lib.ml4_topk_select.restype = C.c_int
    lib.ml4_topk_select.argtypes = [P(ml4_seqs), vp, i64, i32, vp, vp, vp, sz, vp, vp]
    lib.ml4_sparse_mla_decode.restype = C.c_int
    lib.ml4_sparse_mla_decode.argtypes = [P(ml4_seqs), P(ml4_cache), vp, i32, i32, i32, vp, vp,
                                          i32, f32, f32, vp, i32, vp, vp, sz, vp, vp]
    lib.ml4_sparse_mla_decode_e4m3.restype = C.c_int
    lib.ml4_sparse_mla_decode_e4m3.argtypes = [P(ml4_seqs), P(ml4_cache), f32, vp, vp, i32, i32,
                                               vp, vp, i32, f32, f32, vp, i32, vp, vp, sz, vp,
                                               vp]
    lib.ml4_sparse_attn_layer.restype = C.c_int
    lib.ml4_sparse_attn_layer.argtypes = [P(ml4_layer), i32, P(ml4_seqs), P(ml4_cache),
                                          P(ml4_cache), i32, vp, i32, vp, vp, vp, i32,
                                          P(vp), P(vp), vp, i32, vp, vp, sz, vp, vp]
    lib.ml4_sparse_attn_layer_static.restype = C.c_int
    lib.ml4_sparse_attn_layer_static.argtypes = [P(ml4_layer), i32, P(ml4_seqs), P(ml4_cache),
                                                 P(ml4_cache), i32, vp, i32, vp, vp, vp, i32,
                                                 P(vp), P(vp), vp, i32, vp, vp, vp]
    lib.ml4_index_cache_write.restype = C.c_int
    lib.ml4_index_cache_write.argtypes = [P(ml4_cache), i32, vp, i32, i64, vp, vp, vp]
    lib.ml4_latent_cache_write.restype = C.c_int
    lib.ml4_latent_cache_write.argtypes = [P(ml4_cache), i32, vp, i32, vp, i32, i64, vp, vp,
                                           vp]
    lib.ml4_latent_cache_write_e4m3.restype = C.c_int
    lib.ml4_latent_cache_write_e4m3.argtypes = [P(ml4_cache), i32, vp, i32, vp, i32, f32, i64,
                                                vp, vp, vp]
    lib.ml4_window_mla_decode.restype = C.c_int
    lib.ml4_window_mla_decode.argtypes = [P(ml4_seqs), P(ml4_cache), vp, i32, i32, i32, i32,
                                          f32, f32, vp, i32, vp, vp, sz, vp, vp]
    lib.ml4_topk_merge.restype = C.c_int
    lib.ml4_topk_merge.argtypes = [i32, i32, vp, vp, vp, i64, i32, vp, vp, vp, vp]
    lib.ml4_lse_combine.restype = C.c_int
    lib.ml4_lse_combine.argtypes = [i32, i32, i32, i32, vp, vp, vp, i32, vp, vp]
    lib.ml4_probe_read.restype = C.c_int
    lib.ml4_probe_read.argtypes = [vp, sz, vp, vp]
    lib.ml4_probe_mfma.restype = C.c_int
    lib.ml4_probe_mfma.argtypes = [i32, i32, vp, vp]
    if lib.ml4_abi_version() != ML4_ABI_VERSION:
        raise ImportError("libml4dsa.so ABI version mismatch")
    return lib


LIB = _load()


# ---- marshalling helpers
def ptr(x) -> Optional[int]:
    """Device/host address of a torch tensor (or an int / None passthrough)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream=None) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != ML4_OK:
        raise ML4Error(rc, ml4_last_error())
    return rc


def make_seqs(batch) -> ml4_seqs:
    """ml4_seqs over a batch object with device int32 tensors seq_lens, q_start, q_pos,
    block_table and host ints block_size / max_seq_len / max_q_per_seq."""
    s = ml4_seqs()
    s.batch = int(batch.seq_lens.shape[0])
    s.total_q = int(batch.q_pos.shape[0])
    s.max_seq_len = int(batch.max_seq_len)
    s.max_q_per_seq = int(batch.max_q_per_seq)
    s.block_size = int(batch.block_size)
    s.max_blocks_per_seq = int(batch.block_table.shape[1])
    s.seq_lens = ptr(batch.seq_lens)
    s.q_start = ptr(batch.q_start)
    s.q_pos = ptr(batch.q_pos)
    s.block_table = ptr(batch.block_table)
    return s


def make_cache(pool, fmt: int) -> ml4_cache:
    c = ml4_cache()
    c.pool = ptr(pool)
    c.num_blocks = int(pool.shape[0]) if pool is not None else 0
    c.format = fmt
    return c


# ---- the entry points, same names as the C ABI
def ml4_abi_version() -> int:
    return LIB.ml4_abi_version()


def ml4_last_error() -> str:
    return LIB.ml4_last_error().decode()


def ml4_workspace_bytes(entry: int, seqs: ml4_seqs, n_heads: int, top_k: int) -> int:
    return LIB.ml4_workspace_bytes(entry, C.byref(seqs), n_heads, top_k)


def ml4_fault_query(fault, stream=None) -> int:
    bits = C.c_uint32(0)
    rc = LIB.ml4_fault_query(ptr(fault), C.byref(bits), stream_handle(stream))
    if rc not in (ML4_OK, ML4_E_DEVICE_FAULT):
        _check(rc)
    return bits.value


def ml4_indexer_score(seqs, idx_cache, q, q_dtype, q_scale, w, n_heads, ssmax_s, scores,
                      ld_scores, fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_indexer_score(C.byref(seqs), C.byref(idx_cache), ptr(q), q_dtype, ptr(q_scale),
                               ptr(w), n_heads, ssmax_s, ptr(scores), ld_scores, ptr(fault),
                               stream_handle(stream))
    return _check(rc) if check else rc


def ml4_topk_select(seqs, scores, ld_scores, top_k, topk_idx, topk_len, ws=None, ws_bytes=0,
                    fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_topk_select(C.byref(seqs), ptr(scores), ld_scores, top_k, ptr(topk_idx),
                             ptr(topk_len), ptr(ws), ws_bytes, ptr(fault), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_sparse_mla_decode(seqs, kv, q, q_dtype, n_heads, rope_dim, topk_idx, topk_len, top_k,
                          softmax_scale, ssmax_s, out, out_dtype, lse=None, ws=None, ws_bytes=0,
                          fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_sparse_mla_decode(C.byref(seqs), C.byref(kv), ptr(q), q_dtype, n_heads,
                                   rope_dim, ptr(topk_idx), ptr(topk_len), top_k, softmax_scale,
                                   ssmax_s, ptr(out), out_dtype, ptr(lse), ptr(ws), ws_bytes,
                                   ptr(fault), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_sparse_mla_decode_e4m3(seqs, kv, kv_scale, q, q_scale, n_heads, rope_dim, topk_idx,
                               topk_len, top_k, softmax_scale, ssmax_s, out, out_dtype,
                               lse=None, ws=None, ws_bytes=0, fault=None, stream=None,
                               check=True) -> int:
    rc = LIB.ml4_sparse_mla_decode_e4m3(C.byref(seqs), C.byref(kv), kv_scale, ptr(q),
                                        ptr(q_scale), n_heads, rope_dim, ptr(topk_idx),
                                        ptr(topk_len), top_k, softmax_scale, ssmax_s, ptr(out),
                                        out_dtype, ptr(lse), ptr(ws), ws_bytes, ptr(fault),
                                        stream_handle(stream))
    return _check(rc) if check else rc


def ml4_sparse_attn_layer(layers: Sequence[ml4_layer], layer: int, seqs,
                          lat_caches: Sequence[ml4_cache], idx_caches: Sequence[ml4_cache],
                          q_idx, q_idx_dtype, q_idx_scale, w_idx, q_mla, q_mla_dtype,
                          topk_bufs, topk_lens, out, out_dtype, lse=None, ws=None, ws_bytes=0,
                          fault=None, stream=None, check=True) -> int:
    n = len(lat_caches)
    descs = (ml4_layer * n)(*layers)
    lat = (ml4_cache * n)(*lat_caches)
    idx = (ml4_cache * n)(*idx_caches)
    bufs = (C.c_void_p * n)(*[ptr(b) for b in topk_bufs])
    lens = (C.c_void_p * n)(*[ptr(b) for b in topk_lens])
    rc = LIB.ml4_sparse_attn_layer(descs, layer, C.byref(seqs), lat, idx, n, ptr(q_idx),
                                   q_idx_dtype, ptr(q_idx_scale), ptr(w_idx), ptr(q_mla),
                                   q_mla_dtype, bufs, lens, ptr(out), out_dtype, ptr(lse), ptr(ws),
                                   ws_bytes, ptr(fault), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_sparse_attn_layer_static(layers: Sequence[ml4_layer], layer: int, seqs,
                                 lat_caches: Sequence[ml4_cache],
                                 idx_caches: Sequence[ml4_cache], q_idx, q_idx_dtype,
                                 q_idx_scale, w_idx, q_mla, q_mla_dtype, topk_bufs, topk_lens,
                                 out, out_dtype, lse=None, fault=None, stream=None,
                                 check=True) -> int:
    n = len(lat_caches)
    descs = (ml4_layer * n)(*layers)
    lat = (ml4_cache * n)(*lat_caches)
    idx = (ml4_cache * n)(*idx_caches)
    bufs = (C.c_void_p * n)(*[ptr(b) for b in topk_bufs])
    lens = (C.c_void_p * n)(*[ptr(b) for b in topk_lens])
    rc = LIB.ml4_sparse_attn_layer_static(descs, layer, C.byref(seqs), lat, idx, n, ptr(q_idx),
                                          q_idx_dtype, ptr(q_idx_scale), ptr(w_idx),
                                          ptr(q_mla), q_mla_dtype, bufs, lens, ptr(out),
                                          out_dtype, ptr(lse), ptr(fault),
                                          stream_handle(stream))
    return _check(rc) if check else rc


def ml4_index_cache_write(idx_cache, block_size, k, src_dtype, n_tokens, slot_mapping,
                          fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_index_cache_write(C.byref(idx_cache), block_size, ptr(k), src_dtype,
                                   n_tokens, ptr(slot_mapping), ptr(fault),
                                   stream_handle(stream))
    return _check(rc) if check else rc


def ml4_latent_cache_write(lat_cache, block_size, c, src_dtype, k_rope, rope_dim, n_tokens,
                           slot_mapping, fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_latent_cache_write(C.byref(lat_cache), block_size, ptr(c), src_dtype,
                                    ptr(k_rope), rope_dim, n_tokens, ptr(slot_mapping),
                                    ptr(fault), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_latent_cache_write_e4m3(lat_cache, block_size, c, src_dtype, k_rope, rope_dim, kv_scale,
                                n_tokens, slot_mapping, fault=None, stream=None,
                                check=True) -> int:
    rc = LIB.ml4_latent_cache_write_e4m3(C.byref(lat_cache), block_size, ptr(c), src_dtype,
                                         ptr(k_rope), rope_dim, float(kv_scale), n_tokens,
                                         ptr(slot_mapping), ptr(fault), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_topk_merge(rows, n_shards, cand_scores, cand_pos, cand_len, ld_cand, top_k, topk_idx,
                   topk_len, fault=None, stream=None, check=True) -> int:
    rc = LIB.ml4_topk_merge(rows, n_shards, ptr(cand_scores), ptr(cand_pos), ptr(cand_len),
                            ld_cand, top_k, ptr(topk_idx), ptr(topk_len), ptr(fault),
                            stream_handle(stream))
    return _check(rc) if check else rc


def ml4_lse_combine(rows, n_heads, n_shards, head_dim, o_parts, lse_parts, out, out_dtype,
                    lse=None, stream=None, check=True) -> int:
    rc = LIB.ml4_lse_combine(rows, n_heads, n_shards, head_dim, ptr(o_parts), ptr(lse_parts),
                             ptr(out), out_dtype, ptr(lse), stream_handle(stream))
    return _check(rc) if check else rc


def ml4_window_mla_decode(seqs, kv, q, q_dtype, n_heads, rope_dim, window, softmax_scale,
                          ssmax_s, out, out_dtype, lse=None, ws=None, ws_bytes=0, fault=None,
                          stream=None, check=True) -> int:
    rc = LIB.ml4_window_mla_decode(C.byref(seqs), C.byref(kv), ptr(q), q_dtype, n_heads,
                                   rope_dim, window, softmax_scale, ssmax_s, ptr(out),
                                   out_dtype, ptr(lse), ptr(ws), ws_bytes, ptr(fault),
                                   stream_handle(stream))
    return _check(rc) if check else rc


def ml4_probe_read(buf, nbytes, sink, stream=None) -> int:
    return LIB.ml4_probe_read(ptr(buf), nbytes, ptr(sink), stream_handle(stream))


def ml4_probe_mfma(kind, iters, sink, stream=None) -> int:
    return LIB.ml4_probe_mfma(kind, iters, ptr(sink), stream_handle(stream))
