"""Seeded synthetic inputs shaped like the workloads of the pages.

This module only draws and packs random inputs: it holds none of the step's arithmetic
(no scoring, selection or attention).  Both the HIP path and the CPU oracle consume
what it produces; neither is consulted here.  Values are drawn with torch's seeded
generator on the requested device (the CPU for small cases, the GPU for full-size
cases, where billions of values are drawn), so a case is reproducible per
(seed, device).

Recipe (the pages give no activation statistics, so standard normals stand in):
  * indexer key  k ~ N(0,1)^128 per token -> e4m3 codes with one fp32 scale per token
    (scale = amax/448), packed as [128 codes][f32 scale] = 132 B;
  * indexer query q ~ N(0,1) per (row, head) -> e4m3 codes + fp32 scale per (row, head);
    head weights w ~ U(0,1);
  * latent c ~ N(0,1)^512 -> e4m3 codes with one fp32 scale per 128 (amax/448), RoPE part
    kr ~ N(0,1)^64 as bf16, packed as [512 codes][4 x f32][64 x bf16] = 656 B; a NoPE
    layer may fill the RoPE bytes with bf16 NaN to prove they are never read;
  * MLA query ~ N(0,1) as bf16, width 512 + rope_dim;
  * block tables: a seeded random permutation of the physical blocks, dealt to the
    requests in order, so requests interleave in memory;
  * query rows are the trailing positions of each request (decode: p = n-1; verify: the
    last q tokens; prefill: the appended chunk).
fp32 cases (the tiny correctness config) store plain fp32 rows instead.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import torch

E4M3_MAX = 448.0
IDX_DIM = 128
KV_LORA = 512
ROPE_DIM = 64


@dataclass
class Batch:
    seq_lens: torch.Tensor      # int32 [B]
    q_start: torch.Tensor       # int32 [B+1]
    q_pos: torch.Tensor         # int32 [total_q]
    block_table: torch.Tensor   # int32 [B, max_blocks]
    block_size: int
    num_blocks: int
    max_seq_len: int
    max_q_per_seq: int

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_pos.shape[0])

    def to(self, device) -> "Batch":
        return Batch(self.seq_lens.to(device), self.q_start.to(device), self.q_pos.to(device),
                     self.block_table.to(device), self.block_size, self.num_blocks,
                     self.max_seq_len, self.max_q_per_seq)


@dataclass
class LayerInputs:
    """Per-layer caches and queries.  A KV-sharing consumer has lat_pool None; a
    shared-indexer layer has idx_pool / q_idx None."""
    idx_pool: Optional[torch.Tensor] = None     # uint8 [nb, bs, 132] | f32 [nb, bs, 128]
    q_idx: Optional[torch.Tensor] = None        # uint8 [total_q, H_i, 128] | f32
    q_idx_scale: Optional[torch.Tensor] = None  # f32 [total_q, H_i] | None
    w_idx: Optional[torch.Tensor] = None        # f32 [total_q, H_i]
    lat_pool: Optional[torch.Tensor] = None     # uint8 [nb, bs, 656] | f32 [nb, bs, 576]
    q_mla: Optional[torch.Tensor] = None        # bf16 [total_q, H, 512+rope] | f32


@dataclass
class Case:
    name: str
    fmt: str                    # 'fp8' or 'f32'
    batch: Batch
    idx_heads: int
    mla_heads: int
    layers: List[Dict] = field(default_factory=list)   # layer descriptors (plain dicts)
    inputs: Dict[int, LayerInputs] = field(default_factory=dict)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_batch(seed: int, seq_lens: Sequence[int], q_per_seq: Sequence[int], block_size: int,
               extra_blocks: int = 0, device="cpu") -> Batch:
    B = len(seq_lens)
    assert len(q_per_seq) == B
    nblk = [(n + block_size - 1) // block_size for n in seq_lens]
    max_blocks = max(max(nblk), 1)
    num_blocks = sum(nblk) + extra_blocks
    g = _gen(seed, "cpu")
    perm = torch.randperm(max(num_blocks, 1), generator=g).to(torch.int32)
    bt = torch.zeros((B, max_blocks), dtype=torch.int32)
    off = 0
    for b, nb in enumerate(nblk):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    q_start = [0]
    q_pos: List[int] = []
    for n, q in zip(seq_lens, q_per_seq):
        assert 0 <= q <= n
        q_start.append(q_start[-1] + q)
        q_pos.extend(range(n - q, n))
    return Batch(torch.tensor(seq_lens, dtype=torch.int32),
                 torch.tensor(q_start, dtype=torch.int32),
                 torch.tensor(q_pos, dtype=torch.int32), bt, block_size, num_blocks,
                 max(seq_lens) if seq_lens else 0, max(q_per_seq) if q_per_seq else 0).to(device)


def _to_e4m3_codes(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """Pack x / scale as OCP e4m3 codes (torch's round-to-nearest-even cast)."""
    y = (x / scale).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def _amax_scale(x: torch.Tensor) -> torch.Tensor:
    return x.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30) / E4M3_MAX


def make_index_pool(seed: int, num_blocks: int, block_size: int, fmt: str, device="cpu",
                    chunk_tokens: int = 1 << 20) -> torch.Tensor:
    g = _gen(seed, device)
    ntok = num_blocks * block_size
    if fmt == "f32":
        return torch.randn((num_blocks, block_size, IDX_DIM), generator=g, device=device)
    out = torch.empty((ntok, IDX_DIM + 4), dtype=torch.uint8, device=device)
    for s in range(0, ntok, chunk_tokens):
        e = min(ntok, s + chunk_tokens)
        k = torch.randn((e - s, IDX_DIM), generator=g, device=device)
        sc = _amax_scale(k)
        out[s:e, :IDX_DIM] = _to_e4m3_codes(k, sc)
        out[s:e, IDX_DIM:] = sc.to(torch.float32).contiguous().view(torch.uint8)
    return out.view(num_blocks, block_size, IDX_DIM + 4)


def make_latent_pool(seed: int, num_blocks: int, block_size: int, fmt: str,
                     nan_rope: bool = False, device="cpu",
                     chunk_tokens: int = 1 << 19) -> torch.Tensor:
    g = _gen(seed, device)
    ntok = num_blocks * block_size
    if fmt == "f32":
        return torch.randn((num_blocks, block_size, KV_LORA + ROPE_DIM), generator=g,
                           device=device)
    if fmt == "bf16":      # the uncompressed 1,152-byte row: 576 bf16 values
        x = torch.randn((num_blocks, block_size, KV_LORA + ROPE_DIM), generator=g,
                        device=device).to(torch.bfloat16)
        if nan_rope:
            x[..., KV_LORA:] = float("nan")
        return x
    row = KV_LORA + 4 * (KV_LORA // 128) + 2 * ROPE_DIM
    out = torch.empty((ntok, row), dtype=torch.uint8, device=device)
    for s in range(0, ntok, chunk_tokens):
        e = min(ntok, s + chunk_tokens)
        n = e - s
        c = torch.randn((n, KV_LORA // 128, 128), generator=g, device=device)
        sc = _amax_scale(c)                                   # [n, 4, 1]
        out[s:e, :KV_LORA] = _to_e4m3_codes(c, sc).view(n, KV_LORA)
        out[s:e, KV_LORA:KV_LORA + 16] = sc.view(n, 4).to(torch.float32).contiguous().view(torch.uint8)
        rope = torch.randn((n, ROPE_DIM), generator=g, device=device).to(torch.bfloat16)
        if nan_rope:
            rope = torch.full_like(rope, float("nan"))
        out[s:e, KV_LORA + 16:] = rope.contiguous().view(torch.uint8)
    return out.view(num_blocks, block_size, row)


def make_plain_e4m3_pool(seed: int, num_blocks: int, block_size: int, device="cpu",
                         chunk_tokens: int = 1 << 19):
    """Plain E4M3 latent rows (576 codes: 512 latent then 64 RoPE) with one per-tensor
    scale: N(0,1) values quantised with scale 4.5 / 448 (values beyond 4.5 saturate).
    Returns (pool uint8 [num_blocks, block_size, 576], scale)."""
    g = _gen(seed, device)
    ntok = num_blocks * block_size
    scale = 4.5 / E4M3_MAX
    out = torch.empty((ntok, KV_LORA + ROPE_DIM), dtype=torch.uint8, device=device)
    for s in range(0, ntok, chunk_tokens):
        e = min(ntok, s + chunk_tokens)
        x = torch.randn((e - s, KV_LORA + ROPE_DIM), generator=g, device=device)
        out[s:e] = _to_e4m3_codes(x, torch.tensor(scale, device=device))
    return out.view(num_blocks, block_size, KV_LORA + ROPE_DIM), scale


def make_mla_query_fp8(seed: int, total_q: int, heads: int, rope_dim: int, device="cpu"):
    """FP8 MLA queries: E4M3 codes [total_q, heads, 512 + rope_dim] with one amax/448
    scale per (row, head)."""
    g = _gen(seed, device)
    q = torch.randn((total_q, heads, KV_LORA + rope_dim), generator=g, device=device)
    sc = _amax_scale(q)
    return _to_e4m3_codes(q, sc), sc.squeeze(-1).contiguous()


def make_index_query(seed: int, total_q: int, heads: int, fmt: str, device="cpu"):
    g = _gen(seed, device)
    q = torch.randn((total_q, heads, IDX_DIM), generator=g, device=device)
    w = torch.rand((total_q, heads), generator=g, device=device)
    if fmt == "f32":
        return q, None, w
    sc = _amax_scale(q)
    return _to_e4m3_codes(q, sc), sc.squeeze(-1).contiguous(), w


def make_mla_query(seed: int, total_q: int, heads: int, rope_dim: int, fmt: str, device="cpu"):
    g = _gen(seed, device)
    q = torch.randn((total_q, heads, KV_LORA + rope_dim), generator=g, device=device)
    return q if fmt == "f32" else q.to(torch.bfloat16)


def layer_desc(layer: int, *, kv_sharing_target_layer: int = -1, topk_source_layer: int = -1,
               rope_dim: int = ROPE_DIM, top_k: int = 2048, softmax_scale: Optional[float] = None,
               ssmax_s: float = 0.0, idx_ssmax_s: float = 0.0) -> Dict:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(KV_LORA + rope_dim)
    return dict(layer=layer, kv_sharing_target_layer=kv_sharing_target_layer,
                topk_source_layer=topk_source_layer, rope_dim=rope_dim, top_k=top_k,
                softmax_scale=softmax_scale, ssmax_s=ssmax_s, idx_ssmax_s=idx_ssmax_s)


def make_layer_inputs(seed: int, batch: Batch, desc: Dict, fmt: str, idx_heads: int,
                      mla_heads: int, nan_rope: bool = False, device="cpu") -> LayerInputs:
    li = LayerInputs()
    s = seed * 1000 + desc["layer"] * 10
    if desc["topk_source_layer"] < 0:
        li.idx_pool = make_index_pool(s + 1, batch.num_blocks, batch.block_size, fmt, device)
        li.q_idx, li.q_idx_scale, li.w_idx = make_index_query(s + 2, batch.total_q, idx_heads,
                                                              fmt, device)
    if desc["kv_sharing_target_layer"] < 0:
        li.lat_pool = make_latent_pool(s + 3, batch.num_blocks, batch.block_size, fmt,
                                       nan_rope=nan_rope, device=device)
    li.q_mla = make_mla_query(s + 4, batch.total_q, mla_heads, desc["rope_dim"], fmt, device)
    return li


def make_case(name: str, seed: int, *, seq_lens, q_per_seq, block_size: int, fmt: str,
              idx_heads: int, mla_heads: int, layers: List[Dict], extra_blocks: int = 0,
              nan_rope_nope: bool = True, device="cpu") -> Case:
    batch = make_batch(seed, seq_lens, q_per_seq, block_size, extra_blocks, device)
    case = Case(name, fmt, batch, idx_heads, mla_heads, layers)
    for d in layers:
        nan_rope = nan_rope_nope and d["rope_dim"] == 0 and fmt == "fp8"
        case.inputs[d["layer"]] = make_layer_inputs(seed, batch, d, fmt, idx_heads, mla_heads,
                                                    nan_rope, device)
    return case


# ---------------------------------------------------------------------------------------
# The five workloads (full size) and their small same-recipe stand-ins for parity tests.
# ---------------------------------------------------------------------------------------
def config(n: int, device="cpu", seed: Optional[int] = None, scale_down: int = 1) -> Case:
    """n = 1..5.  scale_down > 1 shrinks context lengths and request counts (same recipe,
    same layer modes) for parity runs the oracle finishes in seconds."""
    seed = n if seed is None else seed
    sd = max(1, scale_down)
    if n == 1:
        ctx = max(256, 4096 // sd)
        return make_case("tiny_fp32_decode", seed, seq_lens=[ctx], q_per_seq=[1],
                         block_size=ctx, fmt="f32", idx_heads=16, mla_heads=16,
                         layers=[layer_desc(0, top_k=256)], device=device)
    if n == 2:
        ctx = max(256, 32768 // sd)
        B = max(2, 8 // sd)
        return make_case("decode_b8_32k", seed, seq_lens=[ctx] * B, q_per_seq=[1] * B,
                         block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                         layers=[layer_desc(0)], device=device)
    if n == 3:
        ctx = max(512, 65536 // sd)
        B = max(2, 64 // sd)
        return make_case("verify_64x4_64k", seed, seq_lens=[ctx] * B, q_per_seq=[4] * B,
                         block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                         layers=[layer_desc(0, ssmax_s=0.3),
                                 layer_desc(1, rope_dim=0, ssmax_s=0.3)], device=device)
    if n == 4:
        ctx = max(4096, 1048576 // sd)
        return make_case("decode_b1_1m_3layer", seed, seq_lens=[ctx], q_per_seq=[1],
                         block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                         layers=[layer_desc(0),
                                 layer_desc(1, topk_source_layer=0),
                                 layer_desc(2, kv_sharing_target_layer=0)], device=device)
    if n == 5:
        ctx = max(1024, 32768 // sd)
        q = max(256, 8192 // sd)
        return make_case("prefill_8k_on_24k", seed, seq_lens=[ctx], q_per_seq=[q],
                         block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                         layers=[layer_desc(0)], device=device)
    raise ValueError(n)


def case_to(case: Case, device) -> Case:
    """The same case with every tensor moved to `device` (data movement only)."""
    out = Case(case.name, case.fmt, case.batch.to(device), case.idx_heads, case.mla_heads,
               list(case.layers))
    for l, li in case.inputs.items():
        mv = lambda t: None if t is None else t.to(device)
        out.inputs[l] = LayerInputs(mv(li.idx_pool), mv(li.q_idx), mv(li.q_idx_scale),
                                    mv(li.w_idx), mv(li.lat_pool), mv(li.q_mla))
    return out
