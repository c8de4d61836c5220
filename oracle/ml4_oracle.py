"""Plain fp64 CPU oracle of the DeepSeek-style sparse-attention step of Mistral Large 4.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.  It shares no code with the HIP library.

What is computed, and where the pages state it
----------------------------------------------
Page titles used below:
  [blog]   "vLLM 首日支持 Mistral Large 4：1T 参数 MoE 多模态模型" (best2ai.com translation of
           the vLLM day-0 post)
  [recipe] "mistralai/Mistral-Large-4-1T-A52B — vLLM serving recipe" (recipes.vllm.ai)

1. DSA indexer score  [blog, Highlights; Implementation details › "稀疏 MLA + DSA indexer";
   ROCm implementation details › "AITER 上的 DSA 索引器" (FP8 indexer key with a single
   scale per key, 132 bytes per token per indexer layer)].  The pages name the indexer but
   print no formula; the reading taken is the standard DSA lightning-indexer form
       s[r, t] = m_r * ks[t] * sum_h  w[r,h] * qs[r,h] * ReLU( sum_d q[r,h,d] * k[t,d] )
   over the visible keys t in [0, p_r] (a query sees itself), with m_r the indexer's own
   SSMax multiplier (s_idx * ln(p_r + 1), or 1 when off) [blog, "稀疏 MLA + DSA indexer":
   the indexer has its own SSMax].
2. Exact top-k per query row (k = index_topk = 2048)  [blog, ROCm implementation details ›
   "专用解码" (exact top-2048); Long context › DCP (stable top-k merge; top-k compaction
   with -1 padded slots bounded by topk_length)].  Order: score descending, then lower
   position first; -0 equals +0; NaN ranks below every number.  Output in ascending
   position, padded with -1; length = min(k, p_r + 1).
3. Sparse MLA over the selected rows of the latent cache  [blog, Highlights (KV LoRA rank
   512, RoPE dim 64, top-2048 keys); "稀疏 MLA + DSA indexer" (latent cache, fp8_ds_mla);
   "NoPE、SSMax 和 LeRoPE" (NoPE = RoPE dim 0, same kernel and cache layout; SSMax)]:
       l_t   = sigma_r * ( qa[r,h] . c_t + qr[r,h] . kr_t )
       sigma = softmax_scale * (ssmax_s * ln(p_r + 1) if ssmax_s > 0 else 1)
       o     = sum_t softmax(l)_t c_t         (the latent row is both key and value)
       lse   = max l + ln sum_t exp(l_t - max l)   (natural log)
   Latent row (656 B = the page's fp8_ds_mla size): 512 e4m3 codes, 4 fp32 scales (one per
   128 codes), 64 bf16 RoPE values; c[i] = e4m3(code[i]) * scale[i // 128].
4. Layer modes  [blog, Model architecture (28 layers reuse the nearest preceding indexer
   layer's top-k; NoPE layers 39-71 read layer 35's latent KV); "跨层 KV 共享"
   (kv_sharing_target_layer_name: consumers read the target layer's cache, write none)].
5. Paged addressing: slot = block_table[b][t // block_size] * block_size + t % block_size
   [blog, ROCm implementation details › "AITER 上的稀疏 MLA" (top-2048 positions become
   global cache slots, one entry per query token)].

6. KV-cache writes (the step before the path)  [blog, ROCm implementation details ›
   "AITER 上的 DSA 索引器" (FP8 indexer key with one scale per key, 132 B); "FP8 潜在缓存"
   (fp8_ds_mla: 512 FP8 values with four scales, one per 128, and 64 bf16 RoPE values,
   656 B)].  The pages fix the byte layout but not the quantiser; the reading taken is the
   plain symmetric one: per scale group, scale = amax / 448 (448 = largest E4M3 value) and
   code = E4M3(x / scale) rounded to nearest, ties to even, clamped to +-448; an all-zero
   group gets scale 0 and zero codes.  The code is an integer decided by floating point,
   so it is decided in the kernel's precision: amax, the scale and x / scale are binary32
   operations (each correctly rounded), only the final E4M3 rounding is done here.

7. Split-context merge  [blog, Long context › DCP (each context shard keeps its own top-2048
   candidates; a stable top-k merge over (score, position) pairs -- the order of step 2 --
   gives the row's top-k; partial attentions over disjoint key sets are merged through their
   log-sum-exp)]:
       merge:  top-k of the union of the shards' candidate lists, same order and output form
               as step 2 (ascending position, -1 padded, length min(k, candidates));
       LSE:    M = max_s lse_s,  o = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),
               lse = M + ln sum_s e^(lse_s - M)  (shards with lse = -inf contribute nothing).

8. Second latent layouts  [blog, ROCm implementation details › "FP8 潜在缓存" (the ROCm path
   stores the latent as plain E4M3, 576 B per token with one per-tensor scale, and quantises
   the queries to FP8; the uncompressed row is 576 bf16 values, 1,152 B)]: the plain E4M3
   row is [512 E4M3 latent][64 E4M3 RoPE], value = code * kv_scale; an FP8 query is E4M3
   codes with one fp32 scale per (row, head), value = code * q_scale.  The attention
   formula is step 3's on those values.

Every step is the plain definition, in fp64, in the pages' order; numpy matrix products
serve as the only library primitive.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------------------
# Formats.  Byte counts: [blog, "稀疏 MLA + DSA indexer" (47,136 B per token = 41,328 latent
# + 5,808 indexer); "FP8 潜在缓存" (656 B fp8_ds_mla, 576 B plain E4M3, 1,152 B bf16 per
# token per layer); "AITER 上的 DSA 索引器" (132 B per token per indexer layer)].
# --------------------------------------------------------------------------------------
IDX_DIM = 128
IDX_ROW_FP8 = IDX_DIM + 4            # 128 e4m3 + one fp32 key scale = 132 B
IDX_ROW_F32 = IDX_DIM * 4            # 128 fp32 = 512 B (fp32 test format)
KV_LORA = 512
ROPE_DIM = 64
LAT_SCALE_GROUP = 128
LAT_ROW_FP8 = KV_LORA + 4 * (KV_LORA // LAT_SCALE_GROUP) + 2 * ROPE_DIM   # 656 B
LAT_ROW_F32 = (KV_LORA + ROPE_DIM) * 4                                     # 2,304 B
LAT_ROW_PLAIN_FP8 = KV_LORA + ROPE_DIM                                    # 576 B
LAT_ROW_BF16 = 2 * (KV_LORA + ROPE_DIM)                                   # 1,152 B


def e4m3_value(code: int) -> float:
    """OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; exponent field 0 is subnormal m/8 * 2^-6; max 448."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the top half of an IEEE binary32: value = float32(bits << 16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def decode_f32(raw: np.ndarray) -> np.ndarray:
    """Little-endian fp32 from a trailing byte axis of size 4*n."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    return raw.view("<f4").astype(np.float64)


# --------------------------------------------------------------------------------------
# Sequences and addressing
# --------------------------------------------------------------------------------------
@dataclass
class Seqs:
    """Host copy of a batch: per request b, its cached length seq_lens[b] (including this
    step's tokens), its query rows q_start[b]..q_start[b+1]-1, each query row's absolute
    position q_pos[r] (visible keys 0..q_pos[r]) and its block table."""
    seq_lens: np.ndarray       # [B] int
    q_start: np.ndarray        # [B+1] int
    q_pos: np.ndarray          # [total_q] int
    block_table: np.ndarray    # [B, max_blocks] int
    block_size: int

    @property
    def batch(self) -> int:
        return int(len(self.seq_lens))

    @property
    def total_q(self) -> int:
        return int(self.q_start[-1])

    def request_of(self, r: int) -> int:
        return int(np.searchsorted(self.q_start, r, side="right") - 1)


def slots(seqs: Seqs, b: int, t: np.ndarray) -> np.ndarray:
    """Physical cache slot of logical positions t of request b."""
    t = np.asarray(t, dtype=np.int64)
    bs = seqs.block_size
    return seqs.block_table[b][t // bs].astype(np.int64) * bs + t % bs


# --------------------------------------------------------------------------------------
# Cache row decoders
# --------------------------------------------------------------------------------------
def index_rows_fp8(pool: np.ndarray, s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """pool: uint8 [num_blocks, block_size, 132] -> (k [n,128] values, ks [n] key scales)."""
    flat = pool.reshape(-1, IDX_ROW_FP8)[s]
    k = decode_e4m3(flat[:, :IDX_DIM])
    ks = decode_f32(flat[:, IDX_DIM:IDX_DIM + 4]).reshape(-1)
    return k, ks


def index_rows_f32(pool: np.ndarray, s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """pool: float32 [num_blocks, block_size, 128]; the fp32 format has no key scale."""
    flat = pool.reshape(-1, IDX_DIM)[s].astype(np.float64)
    return flat, np.ones(len(s), dtype=np.float64)


def latent_rows_fp8(pool: np.ndarray, s: np.ndarray, rope_dim: int
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """pool: uint8 [num_blocks, block_size, 656] -> (c [n,512] dequantised latent,
    kr [n,rope_dim] RoPE part).  With rope_dim == 0 the RoPE bytes are never read."""
    flat = pool.reshape(-1, LAT_ROW_FP8)[s]
    codes = decode_e4m3(flat[:, :KV_LORA])
    ngrp = KV_LORA // LAT_SCALE_GROUP
    scales = decode_f32(flat[:, KV_LORA:KV_LORA + 4 * ngrp]).reshape(-1, ngrp)
    c = codes * np.repeat(scales, LAT_SCALE_GROUP, axis=1)
    if rope_dim:
        rb = np.ascontiguousarray(flat[:, KV_LORA + 4 * ngrp:KV_LORA + 4 * ngrp + 2 * rope_dim])
        kr = decode_bf16(rb.view("<u2"))
    else:
        kr = np.zeros((len(s), 0))
    return c, kr


def latent_rows_f32(pool: np.ndarray, s: np.ndarray, rope_dim: int
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """pool: float32 [num_blocks, block_size, 576] (512 latent then 64 RoPE)."""
    flat = pool.reshape(-1, KV_LORA + ROPE_DIM)[s].astype(np.float64)
    return flat[:, :KV_LORA], flat[:, KV_LORA:KV_LORA + rope_dim]


def latent_rows_bf16(pool: np.ndarray, s: np.ndarray, rope_dim: int
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """pool: uint16 bf16 bits [num_blocks, block_size, 576] (512 latent then 64 RoPE) -- the
    uncompressed 1,152-B row [blog, "FP8 潜在缓存"].  With rope_dim == 0 the RoPE values are
    never read."""
    flat = pool.reshape(-1, KV_LORA + ROPE_DIM)[s]
    return decode_bf16(flat[:, :KV_LORA]), decode_bf16(flat[:, KV_LORA:KV_LORA + rope_dim])


def latent_rows_e4m3(pool: np.ndarray, s: np.ndarray, rope_dim: int, kv_scale: float
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """pool: uint8 [num_blocks, block_size, 576] plain E4M3 rows (512 latent then 64 RoPE),
    one per-tensor scale.  With rope_dim == 0 the RoPE codes are never read."""
    flat = pool.reshape(-1, KV_LORA + ROPE_DIM)[s]
    c = decode_e4m3(flat[:, :KV_LORA]) * float(kv_scale)
    kr = decode_e4m3(flat[:, KV_LORA:KV_LORA + rope_dim]) * float(kv_scale)
    return c, kr


def window_positions(q_pos: np.ndarray, window: int) -> Tuple[np.ndarray, np.ndarray]:
    """Sliding-window selection [blog, Long context (DSpark draft layers: a 2,048-token
    window)]: row r attends to max(0, p_r - window + 1) .. p_r.  Returned in the top-k list
    form (idx [rows][window] ascending, -1 padded; len)."""
    idx = np.full((len(q_pos), window), -1, dtype=np.int64)
    ln = np.zeros(len(q_pos), dtype=np.int64)
    for r, p in enumerate(q_pos):
        lo = max(0, int(p) - window + 1)
        n = int(p) - lo + 1
        idx[r, :n] = np.arange(lo, int(p) + 1)
        ln[r] = n
    return idx, ln


def ssmax_multiplier(ssmax_s: float, pos: int) -> float:
    """SSMax logit multiplier s * ln(n) with n = p + 1 visible keys; 1 when s <= 0."""
    return ssmax_s * math.log(pos + 1) if ssmax_s > 0 else 1.0


# --------------------------------------------------------------------------------------
# 1. Indexer scores
# --------------------------------------------------------------------------------------
def indexer_scores(seqs: Seqs, pool: np.ndarray, fmt: str, q: np.ndarray,
                   q_scale: Optional[np.ndarray], w: np.ndarray, ssmax_s: float,
                   ld: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Scores [len(rows), ld] in fp64; -inf for t > q_pos[r].

    fmt 'fp8': q is uint8 e4m3 codes [total_q, H, 128], pool uint8 [nb, bs, 132].
    fmt 'f32': q is float32 [total_q, H, 128], pool float32 [nb, bs, 128].
    q_scale [total_q, H] (None = 1), w [total_q, H].
    """
    if fmt not in ("fp8", "f32"):
        raise ValueError(f"indexer_scores: unknown index format {fmt!r}")
    rows = range(seqs.total_q) if rows is None else rows
    out = np.full((len(rows), ld), -np.inf)
    for i, r in enumerate(rows):
        b = seqs.request_of(r)
        p = int(seqs.q_pos[r])
        t = np.arange(p + 1)
        s = slots(seqs, b, t)
        if fmt == "fp8":
            k, ks = index_rows_fp8(pool, s)
            qv = decode_e4m3(q[r])                      # [H, 128]
        else:
            k, ks = index_rows_f32(pool, s)
            qv = np.asarray(q[r], dtype=np.float64)
        qs = np.ones(qv.shape[0]) if q_scale is None else np.asarray(q_scale[r], np.float64)
        dots = qv @ k.T                                  # [H, p+1]: q_h . k_t
        relu = np.maximum(dots, 0.0)
        weighted = (np.asarray(w[r], np.float64) * qs) @ relu   # sum over heads
        out[i, :p + 1] = ssmax_multiplier(ssmax_s, p) * ks * weighted
    return out


# --------------------------------------------------------------------------------------
# 2. Exact top-k
# --------------------------------------------------------------------------------------
def topk_row(scores: np.ndarray, pos: int, top_k: int) -> Tuple[np.ndarray, int]:
    """Exact top-k over candidates t in [0, pos]: (idx[top_k] ascending, -1 padded; len)."""
    cand = np.asarray(scores[:pos + 1], dtype=np.float64)
    t = np.arange(pos + 1)
    nan = np.isnan(cand)
    key = np.where(nan, 0.0, -cand)          # -(-0.0) == 0.0 compares equal to -(0.0)
    order = np.lexsort((t, key, nan))        # primary: not-NaN first; then score desc; then t asc
    n = min(top_k, pos + 1)
    sel = np.sort(t[order[:n]])
    out = np.full(top_k, -1, dtype=np.int64)
    out[:n] = sel
    return out, n


def topk_select(scores: np.ndarray, q_pos: np.ndarray, top_k: int
                ) -> Tuple[np.ndarray, np.ndarray]:
    idx = np.full((len(q_pos), top_k), -1, dtype=np.int64)
    ln = np.zeros(len(q_pos), dtype=np.int64)
    for r, p in enumerate(q_pos):
        idx[r], ln[r] = topk_row(scores[r], int(p), top_k)
    return idx, ln


# --------------------------------------------------------------------------------------
# 3. Sparse MLA (two-pass softmax, not online)
# --------------------------------------------------------------------------------------
def sparse_mla(seqs: Seqs, pool: np.ndarray, fmt: str, q: np.ndarray, rope_dim: int,
               topk_idx: np.ndarray, topk_len: np.ndarray, softmax_scale: float,
               ssmax_s: float, rows: Optional[Sequence[int]] = None,
               q_scale: Optional[np.ndarray] = None, kv_scale: float = 1.0
               ) -> Tuple[np.ndarray, np.ndarray]:
    """o [len(rows), H, 512] and lse [len(rows), H] in fp64.

    fmt 'fp8': pool uint8 [nb, bs, 656]; q uint16 bf16 bits [total_q, H, 512 + rope_dim].
    fmt 'bf16': pool uint16 bf16 bits [nb, bs, 576]; q as for 'fp8'.
    fmt 'e4m3': pool uint8 [nb, bs, 576] plain E4M3 rows times kv_scale; q uint8 E4M3 codes
                [total_q, H, 512 + rope_dim] times q_scale [total_q, H].
    fmt 'f32': pool float32 [nb, bs, 576]; q float32 [total_q, H, 512 + rope_dim].
    topk_idx holds logical positions; entries past topk_len[r] are ignored.  Any other
    format is refused.
    """
    if fmt not in ("fp8", "bf16", "e4m3", "f32"):
        raise ValueError(f"sparse_mla: unknown latent format {fmt!r}")
    if fmt == "e4m3" and q_scale is None:
        raise ValueError("sparse_mla: the 'e4m3' format needs q_scale")
    rows = range(seqs.total_q) if rows is None else rows
    H = q.shape[1]
    o = np.zeros((len(rows), H, KV_LORA))
    lse = np.full((len(rows), H), -np.inf)
    for i, r in enumerate(rows):
        b = seqs.request_of(r)
        n = int(topk_len[r])
        if n == 0:
            continue
        t = np.asarray(topk_idx[r][:n], dtype=np.int64)
        s = slots(seqs, b, t)
        if fmt == "fp8":
            c, kr = latent_rows_fp8(pool, s, rope_dim)
            qv = decode_bf16(q[r])
        elif fmt == "bf16":
            c, kr = latent_rows_bf16(pool, s, rope_dim)
            qv = decode_bf16(q[r])
        elif fmt == "e4m3":
            c, kr = latent_rows_e4m3(pool, s, rope_dim, kv_scale)
            qv = decode_e4m3(q[r]) * np.asarray(q_scale[r], dtype=np.float64)[:, None]
        else:
            c, kr = latent_rows_f32(pool, s, rope_dim)
            qv = np.asarray(q[r], dtype=np.float64)
        qa, qr = qv[:, :KV_LORA], qv[:, KV_LORA:KV_LORA + rope_dim]
        sigma = softmax_scale * ssmax_multiplier(ssmax_s, int(seqs.q_pos[r]))
        logits = sigma * (qa @ c.T + qr @ kr.T)          # [H, n]
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        z = e.sum(axis=1, keepdims=True)
        o[i] = (e / z) @ c
        lse[i] = m[:, 0] + np.log(z[:, 0])
    return o, lse


def dense_mla(seqs: Seqs, pool: np.ndarray, fmt: str, q: np.ndarray, rope_dim: int,
              softmax_scale: float, ssmax_s: float,
              rows: Optional[Sequence[int]] = None, q_scale: Optional[np.ndarray] = None,
              kv_scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray]:
    """Dense MLA over every visible key t in [0, q_pos[r]]: softmax(sigma Q K^T) V with
    K = [c | kr] and V = c, written as whole-matrix products.  Equals sparse_mla whenever
    the selection holds every visible key (top_k >= context).

    Formats and query types as sparse_mla: 'fp8' (656-B rows, bf16 q), 'bf16' (1,152-B
    rows, bf16 q), 'e4m3' (576-B plain E4M3 rows times kv_scale, E4M3 q times q_scale
    [total_q, H]), 'f32' (fp32 rows and q).  Any other format is refused."""
    if fmt not in ("fp8", "bf16", "e4m3", "f32"):
        raise ValueError(f"dense_mla: unknown latent format {fmt!r}")
    if fmt == "e4m3" and q_scale is None:
        raise ValueError("dense_mla: the 'e4m3' format needs q_scale")
    rows = range(seqs.total_q) if rows is None else rows
    H = q.shape[1]
    o = np.zeros((len(rows), H, KV_LORA))
    lse = np.zeros((len(rows), H))
    for i, r in enumerate(rows):
        b = seqs.request_of(r)
        p = int(seqs.q_pos[r])
        sl = slots(seqs, b, np.arange(p + 1))
        if fmt == "fp8":
            c, kr = latent_rows_fp8(pool, sl, rope_dim)
            qv = decode_bf16(q[r])
        elif fmt == "bf16":
            c, kr = latent_rows_bf16(pool, sl, rope_dim)
            qv = decode_bf16(q[r])
        elif fmt == "e4m3":
            c, kr = latent_rows_e4m3(pool, sl, rope_dim, kv_scale)
            qv = decode_e4m3(q[r]) * np.asarray(q_scale[r], dtype=np.float64)[:, None]
        else:
            c, kr = latent_rows_f32(pool, sl, rope_dim)
            qv = np.asarray(q[r], np.float64)
        K = np.concatenate([c, kr], axis=1)               # [n, 512 + rope]
        Q = qv[:, :KV_LORA + rope_dim]
        S = softmax_scale * ssmax_multiplier(ssmax_s, p) * (Q @ K.T)
        mx = S.max(axis=1)
        P = np.exp(S - mx[:, None])
        Z = P.sum(axis=1)
        o[i] = (P @ c) / Z[:, None]
        lse[i] = mx + np.log(Z)
    return o, lse


# --------------------------------------------------------------------------------------
# 4. Layer modes
# --------------------------------------------------------------------------------------
@dataclass
class Layer:
    layer: int
    kv_sharing_target_layer: int = -1   # -1: reads its own latent cache
    topk_source_layer: int = -1         # -1: runs its own indexer
    rope_dim: int = ROPE_DIM            # 0 for a NoPE layer
    top_k: int = 2048
    softmax_scale: float = 1.0 / math.sqrt(KV_LORA + ROPE_DIM)
    ssmax_s: float = 0.0
    idx_ssmax_s: float = 0.0


def layer_step(L: Layer, seqs: Seqs, fmt: str, lat_pools: Dict[int, np.ndarray],
               idx_pools: Dict[int, np.ndarray], q_idx, q_idx_scale, w_idx, q_mla,
               topk_store: Dict[int, Tuple[np.ndarray, np.ndarray]], ld: int,
               rows: Optional[Sequence[int]] = None):
    """One layer: indexer -> top-k -> sparse MLA, honouring the layer modes.

    A shared-indexer layer reads topk_store[topk_source_layer] and runs no indexer; a
    KV-sharing consumer reads lat_pools[kv_sharing_target_layer].  An indexer-owning
    layer records its (topk_idx, topk_len) in topk_store[layer]."""
    rows = list(range(seqs.total_q)) if rows is None else list(rows)
    lat = lat_pools[L.kv_sharing_target_layer if L.kv_sharing_target_layer >= 0 else L.layer]
    if L.topk_source_layer >= 0:
        idx, ln = topk_store[L.topk_source_layer]
    else:
        sc = indexer_scores(seqs, idx_pools[L.layer], fmt, q_idx, q_idx_scale, w_idx,
                            L.idx_ssmax_s, ld, rows)
        idx = np.full((seqs.total_q, L.top_k), -1, dtype=np.int64)
        ln = np.zeros(seqs.total_q, dtype=np.int64)
        for i, r in enumerate(rows):
            idx[r], ln[r] = topk_row(sc[i], int(seqs.q_pos[r]), L.top_k)
        topk_store[L.layer] = (idx, ln)
    o, lse = sparse_mla(seqs, lat, fmt, q_mla, L.rope_dim, idx, ln, L.softmax_scale,
                        L.ssmax_s, rows)
    return o, lse, idx, ln


# --------------------------------------------------------------------------------------
# Model-level byte arithmetic [blog, Model architecture; "稀疏 MLA + DSA indexer";
# "跨层 KV 共享"; "FP8 潜在缓存"] -- used to pin the row formats above.
# --------------------------------------------------------------------------------------
N_LAYERS = 72
KV_CONSUMERS = tuple(range(39, 72, 4))   # NoPE layers 39..71 read layer 35's latent KV
N_INDEX_SHARERS = 28                     # layers reusing the nearest preceding indexer


def nope_layers() -> Tuple[int, ...]:
    """Every fourth layer is NoPE: 3, 7, ..., 71."""
    return tuple(l for l in range(N_LAYERS) if l % 4 == 3)


def kv_bytes_per_token(latent_row: int, index_row: int = IDX_ROW_FP8) -> int:
    owners = N_LAYERS - len(KV_CONSUMERS)
    indexers = N_LAYERS - N_INDEX_SHARERS
    return owners * latent_row + indexers * index_row


# --------------------------------------------------------------------------------------
# 6. KV-cache writes: quantise and pack rows  [blog, "AITER 上的 DSA 索引器"; "FP8 潜在缓存"]
# --------------------------------------------------------------------------------------
E4M3_MAX = 448.0


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """binary32 values already inside [-448, 448] -> OCP E4M3 codes, round to nearest with
    ties to even.  The grid is 2^-9 steps below 2^-6 (subnormals) and 8 steps per binade
    above; the sign of zero is kept."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    assert np.all(np.isfinite(v)) and np.all(np.abs(v) <= E4M3_MAX)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal binade: value = m * 2^-9, m in 0..8 (m = 8 is the smallest normal, code 8)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        m, e = np.frexp(a[nrm])                  # a = m * 2^e, m in [0.5, 1)
        e = e - 1                                # a = (2m) * 2^e, 2m in [1, 2)
        q = np.rint(2.0 * m * 8.0).astype(np.int64)   # 8 .. 16 (ties to even)
        up = q == 16
        e = np.where(up, e + 1, e)
        q = np.where(up, 8, q)
        code[nrm] = ((e + 7) << 3) | (q - 8)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def _quantise_group(x32: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """One scale group (binary32 values) -> (codes, scale)."""
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0.0)
    scale = np.float32(amax / np.float32(E4M3_MAX))
    if scale == 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(0.0)
    v = (x32 / scale).astype(np.float32)                 # binary32 division
    v = np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return encode_e4m3(v), scale


def quantise_index_rows(k32: np.ndarray) -> np.ndarray:
    """[n][128] binary32 keys -> [n][132] rows: 128 E4M3 codes then the fp32 key scale."""
    k32 = np.asarray(k32, dtype=np.float32)
    out = np.zeros((k32.shape[0], IDX_ROW_FP8), dtype=np.uint8)
    for i in range(k32.shape[0]):
        codes, sc = _quantise_group(k32[i])
        out[i, :IDX_DIM] = codes
        out[i, IDX_DIM:] = np.frombuffer(np.float32(sc).tobytes(), dtype=np.uint8)
    return out


def quantise_latent_rows(c32: np.ndarray, rope_bf16_bits: Optional[np.ndarray]) -> np.ndarray:
    """[n][512] binary32 latents (+ [n][64] bf16 RoPE bits, or None) -> [n][656] rows:
    512 E4M3 codes, four fp32 scales (one per 128 codes), 64 bf16 RoPE values (left zero
    here when None: a NoPE write does not touch those bytes)."""
    c32 = np.asarray(c32, dtype=np.float32)
    out = np.zeros((c32.shape[0], LAT_ROW_FP8), dtype=np.uint8)
    ng = KV_LORA // LAT_SCALE_GROUP
    for i in range(c32.shape[0]):
        for g in range(ng):
            codes, sc = _quantise_group(c32[i, g * LAT_SCALE_GROUP:(g + 1) * LAT_SCALE_GROUP])
            out[i, g * LAT_SCALE_GROUP:(g + 1) * LAT_SCALE_GROUP] = codes
            out[i, KV_LORA + 4 * g:KV_LORA + 4 * g + 4] = np.frombuffer(
                np.float32(sc).tobytes(), dtype=np.uint8)
        if rope_bf16_bits is not None:
            out[i, KV_LORA + 4 * ng:] = np.frombuffer(
                np.asarray(rope_bf16_bits[i], dtype="<u2").tobytes(), dtype=np.uint8)
    return out


def encode_bf16(v: np.ndarray) -> np.ndarray:
    """Finite binary32 values -> bfloat16 bits, round to nearest with ties to even on the
    16 dropped bits of the IEEE binary32 pattern (a carry into the exponent is the correct
    rounding up to the next binade)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    assert np.all(np.isfinite(np.asarray(v, dtype=np.float32)))
    keep = u >> 16
    rest = u & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def pack_latent_rows_bf16(c32: np.ndarray, rope_bf16_bits: Optional[np.ndarray]) -> np.ndarray:
    """Second layout, write side [blog, ROCm implementation details › "FP8 潜在缓存" (the
    uncompressed 1,152-B row)]: [n][512] binary32 latents (+ [n][64] bf16 RoPE bits, or None)
    -> [n][576] bf16 bits, latents rounded to nearest even, RoPE copied (left zero when None:
    a NoPE write does not touch those values)."""
    c32 = np.asarray(c32, dtype=np.float32)
    out = np.zeros((c32.shape[0], KV_LORA + ROPE_DIM), dtype=np.uint16)
    out[:, :KV_LORA] = encode_bf16(c32)
    if rope_bf16_bits is not None:
        out[:, KV_LORA:] = np.asarray(rope_bf16_bits, dtype=np.uint16)
    return out


def quantise_latent_rows_e4m3(c32: np.ndarray, rope32: Optional[np.ndarray], kv_scale: float
                              ) -> np.ndarray:
    """Second layout, write side [blog, ROCm implementation details › "FP8 潜在缓存" (all 576
    dims in E4M3 with one per-tensor scale)]: code = E4M3(x / kv_scale) in binary32, rounded
    to nearest even and clamped to +-448, for the 512 latents and (when given) the 64 RoPE
    values; [n][576] codes, RoPE codes left zero when None."""
    scale = np.float32(kv_scale)
    def q(x):
        v = (np.asarray(x, dtype=np.float32) / scale).astype(np.float32)   # binary32 division
        return encode_e4m3(np.clip(v, -E4M3_MAX, E4M3_MAX).astype(np.float32))
    c32 = np.asarray(c32, dtype=np.float32)
    out = np.zeros((c32.shape[0], KV_LORA + ROPE_DIM), dtype=np.uint8)
    out[:, :KV_LORA] = q(c32)
    if rope32 is not None:
        out[:, KV_LORA:] = q(rope32)
    return out


# --------------------------------------------------------------------------------------
# 7. Split-context merge  [blog, Long context › DCP]
# --------------------------------------------------------------------------------------
def topk_merge(cand_scores: np.ndarray, cand_pos: np.ndarray, cand_len: np.ndarray,
               top_k: int) -> Tuple[np.ndarray, int]:
    """cand_scores / cand_pos: [S][k_s] per-shard candidate lists (entries past cand_len[s]
    are ignored); positions are distinct.  Top-k of their union in the order of step 2:
    (idx[top_k] ascending, -1 padded; len)."""
    sc, ps = [], []
    for s_ in range(len(cand_len)):
        n = int(cand_len[s_])
        sc.append(np.asarray(cand_scores[s_][:n], dtype=np.float64))
        ps.append(np.asarray(cand_pos[s_][:n], dtype=np.int64))
    sc = np.concatenate(sc) if sc else np.zeros(0)
    ps = np.concatenate(ps) if ps else np.zeros(0, dtype=np.int64)
    assert len(np.unique(ps)) == len(ps)
    nan = np.isnan(sc)
    key = np.where(nan, 0.0, -sc)
    order = np.lexsort((ps, key, nan))
    n = min(top_k, len(ps))
    out = np.full(top_k, -1, dtype=np.int64)
    out[:n] = np.sort(ps[order[:n]])
    return out, n


def lse_combine(o_parts: np.ndarray, lse_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """o_parts [S][H][D], lse_parts [S][H] (natural log; -inf = empty shard) ->
    (o [H][D], lse [H])."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    M = np.max(lse_parts, axis=0)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - Ms[None, :]), 0.0)
    den = w.sum(axis=0)
    o = np.einsum("sh,shd->hd", w, o_parts) / np.where(den > 0, den, 1.0)[:, None]
    o[~live] = 0.0
    lse = np.where(live, Ms + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    return o, lse
