"""Device buffers and per-layer calls over a synthetic case (marshalling only).

A CaseRunner owns the outputs, top-k buffers, workspace and fault word of a case whose
inputs already sit in device memory, and runs its layers either through the fused entry
ml4_sparse_attn_layer or through the three separate entries (optionally bracketing each
with HIP events on the launch stream).
"""

from __future__ import annotations

from typing import Dict, List, Optional

import torch

from . import ml4dsa as M
from .synth import Case

_FMT = {
    "fp8": (M.ML4_IDX_FP8_132, M.ML4_LAT_FP8_656, M.ML4_FP8_E4M3, M.ML4_BF16, torch.bfloat16),
    "f32": (M.ML4_IDX_F32, M.ML4_LAT_F32, M.ML4_F32, M.ML4_F32, torch.float32),
}


def _r256(x: int) -> int:
    return (x + 255) // 256 * 256


class CaseRunner:
    def __init__(self, case: Case):
        self.case = case
        b = case.batch
        dev = b.seq_lens.device
        assert dev.type == "cuda", "inputs must be in device memory"
        self.dev = dev
        self.seqs = M.make_seqs(b)
        idx_fmt, lat_fmt, self.qi_dtype, self.qm_dtype, out_t = _FMT[case.fmt]
        self.n_layers = max(d["layer"] for d in case.layers) + 1
        empty = M.ml4_cache()
        self.lat_caches: List[M.ml4_cache] = [M.ml4_cache() for _ in range(self.n_layers)]
        self.idx_caches: List[M.ml4_cache] = [M.ml4_cache() for _ in range(self.n_layers)]
        self.desc: Dict[int, M.ml4_layer] = {}
        self.topk_idx: Dict[int, torch.Tensor] = {}
        self.topk_len: Dict[int, torch.Tensor] = {}
        self.out: Dict[int, torch.Tensor] = {}
        self.lse: Dict[int, torch.Tensor] = {}
        T = b.total_q
        ws = 0
        for d in case.layers:
            l = d["layer"]
            li = case.inputs[l]
            if li.lat_pool is not None:
                self.lat_caches[l] = M.make_cache(li.lat_pool, lat_fmt)
            if li.idx_pool is not None:
                self.idx_caches[l] = M.make_cache(li.idx_pool, idx_fmt)
            L = M.ml4_layer()
            L.layer = l
            L.kv_sharing_target_layer = d["kv_sharing_target_layer"]
            L.topk_source_layer = d["topk_source_layer"]
            L.rope_dim = d["rope_dim"]
            L.top_k = d["top_k"]
            L.idx_heads = case.idx_heads
            L.mla_heads = case.mla_heads
            L.softmax_scale = d["softmax_scale"]
            L.ssmax_s = d["ssmax_s"]
            L.idx_ssmax_s = d["idx_ssmax_s"]
            self.desc[l] = L
            if d["topk_source_layer"] < 0:
                self.topk_idx[l] = torch.full((T, d["top_k"]), -7, dtype=torch.int32, device=dev)
                self.topk_len[l] = torch.full((T,), -7, dtype=torch.int32, device=dev)
            self.out[l] = torch.empty((T, case.mla_heads, 512), dtype=out_t, device=dev)
            self.lse[l] = torch.empty((T, case.mla_heads), dtype=torch.float32, device=dev)
            ws = max(ws, M.ml4_workspace_bytes(M.ML4_ENTRY_LAYER, self.seqs, case.mla_heads,
                                               d["top_k"]))
        # descriptors of every layer index, in order (an index the case does not run gets
        # an owner descriptor that no call names)
        self.layers: List[M.ml4_layer] = []
        for i in range(self.n_layers):
            if i in self.desc:
                self.layers.append(self.desc[i])
            else:
                D = M.ml4_layer()
                D.layer, D.kv_sharing_target_layer, D.topk_source_layer = i, -1, -1
                self.layers.append(D)
        self.ld = (b.max_seq_len + 3) // 4 * 4
        self.ws_bytes = max(ws, 256)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.fault = torch.zeros(1, dtype=torch.int32, device=dev)
        self._empty = empty

    # views into the workspace used by the separate-entry path
    def scores_view(self) -> torch.Tensor:
        T = self.case.batch.total_q
        return self.ws[: T * self.ld * 4].view(torch.float32).view(T, self.ld)

    def _topk_ws(self, top_k: int):
        off = _r256(self.case.batch.total_q * self.ld * 4)
        n = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, self.seqs, 0, top_k)
        return (self.ws[off:].data_ptr() if n else None), n, off + n

    def _mla_ws(self, top_k: int):
        _, _, off = self._topk_ws(top_k)
        n = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, self.seqs, self.case.mla_heads, top_k)
        return (self.ws[off:].data_ptr() if n else None), n

    def topk_of(self, l: int):
        d = self.desc[l]
        src = d.topk_source_layer if d.topk_source_layer >= 0 else l
        return self.topk_idx[src], self.topk_len[src]

    def lat_pool_of(self, l: int):
        d = self.desc[l]
        return self.lat_caches[d.kv_sharing_target_layer if d.kv_sharing_target_layer >= 0 else l]

    def run_layer_fused(self, l: int, stream=None):
        li = self.case.inputs[l]
        bufs = [self.topk_idx.get(i) for i in range(self.n_layers)]
        lens = [self.topk_len.get(i) for i in range(self.n_layers)]
        M.ml4_sparse_attn_layer(self.layers, l, self.seqs, self.lat_caches, self.idx_caches,
                                li.q_idx,
                                self.qi_dtype, li.q_idx_scale, li.w_idx, li.q_mla,
                                self.qm_dtype, bufs, lens, self.out[l], self.qm_dtype,
                                self.lse[l], self.ws, self.ws_bytes, self.fault, stream)

    def run_layer_static(self, l: int, stream=None):
        """The fused layer through the no-allocation entry (the library's fixed scratch
        instead of this runner's workspace)."""
        li = self.case.inputs[l]
        bufs = [self.topk_idx.get(i) for i in range(self.n_layers)]
        lens = [self.topk_len.get(i) for i in range(self.n_layers)]
        M.ml4_sparse_attn_layer_static(self.layers, l, self.seqs, self.lat_caches,
                                       self.idx_caches, li.q_idx, self.qi_dtype,
                                       li.q_idx_scale, li.w_idx, li.q_mla, self.qm_dtype, bufs,
                                       lens, self.out[l], self.qm_dtype, self.lse[l],
                                       self.fault, stream)

    def run_layer_split(self, l: int, events: Optional[List] = None, stream=None):
        """indexer -> top-k -> MLA through the separate entries.  events, when given, is a
        list of 4 torch.cuda.Event recorded on the launch stream around the three calls."""
        li = self.case.inputs[l]
        L = self.desc[l]
        st = stream if stream is not None else torch.cuda.current_stream()
        rec = (lambda i: events[i].record(st)) if events else (lambda i: None)
        rec(0)
        if L.topk_source_layer < 0:
            sc = self.scores_view()
            M.ml4_indexer_score(self.seqs, self.idx_caches[l], li.q_idx, self.qi_dtype,
                                li.q_idx_scale, li.w_idx, L.idx_heads, L.idx_ssmax_s, sc,
                                self.ld, self.fault, st)
            rec(1)
            wsp, wsn, _ = self._topk_ws(L.top_k)
            M.ml4_topk_select(self.seqs, sc, self.ld, L.top_k, self.topk_idx[l],
                              self.topk_len[l], wsp, wsn, self.fault, st)
            rec(2)
        else:
            rec(1)
            rec(2)
        idx, ln = self.topk_of(l)
        wsp, wsn = self._mla_ws(L.top_k)
        M.ml4_sparse_mla_decode(self.seqs, self.lat_pool_of(l), li.q_mla, self.qm_dtype,
                                L.mla_heads, L.rope_dim, idx, ln, L.top_k, L.softmax_scale,
                                L.ssmax_s, self.out[l], self.qm_dtype, self.lse[l], wsp, wsn,
                                self.fault, st)
        rec(3)

    def run_step(self, fused: bool = True, stream=None):
        for d in self.case.layers:
            if fused:
                self.run_layer_fused(d["layer"], stream)
            else:
                self.run_layer_split(d["layer"], stream=stream)

    def fault_bits(self) -> int:
        return M.ml4_fault_query(self.fault)
