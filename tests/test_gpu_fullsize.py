"""Parity at the five workloads' full sizes, on the inputs and through the entries the bench
times (MI355X only): the seeded workload is generated on the GPU exactly as the bench does
and each layer runs through the separate entries with the bench's launch configuration.
On sampled query rows the oracle recomputes, one row at a time.  The sample holds every row
of a small batch, else whole groups of four consecutive rows (the first, a middle and the
last group: every slot of a multi-row indexer work-group) and, for long prefill rows, 16
rows spread evenly over the causal range (so over several key chunks):

* indexer scores over every visible key, within 2e-5 of the row's largest |score| (fp32
  accumulation of exact e4m3 products), -inf past the row's position;
* the top-k list, bit-exact against the oracle's exact selection on the kernel's own fp32
  scores (the integer decision taken in the kernel's precision), and against the oracle's
  fp64 scores up to near-ties (tests/compare.py);
* attention output and LSE, |d| <= 2e-3 + 1e-2 |ref|, with the layer modes resolved as the
  bench runs them (shared-indexer layers reuse the owner's top-k, consumers read the
  owner's latent cache);
* end to end: attention on the oracle's own top-k set (from its fp64 scores) against the
  GPU output, reported per layer; where the two sets are equal it must meet the attention
  bound as well.
"""

import numpy as np
import pytest
import torch

import oracle as O
from tests.compare import batch_np, check_close, check_topk_rows, t_np

pytestmark = pytest.mark.gpu

M = pytest.importorskip("sparse_attention_decode_dsa_amd.ml4dsa")
from sparse_attention_decode_dsa_amd import synth  # noqa: E402
from sparse_attention_decode_dsa_amd.runner import CaseRunner  # noqa: E402

DEV = "cuda:0"
SCORE_RTOL = 2e-5


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _say(msg):
    print(msg, flush=True)


def _sample_rows(total_q):
    if total_q <= 8:
        return list(range(total_q))
    mid = (total_q // 2) & ~3
    rows = set(range(4)) | set(range(mid, mid + 4)) | set(range(total_q - 4, total_q))
    if total_q >= 1024:
        rows |= {int(round(x)) for x in np.linspace(0, total_q - 1, 16)}
    return sorted(rows)


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_workload_sampled_rows(config):
    case = synth.config(config, device=DEV)          # the bench's inputs (same seed)
    torch.cuda.synchronize()
    run = CaseRunner(case)
    s = batch_np(case.batch)
    rows = _sample_rows(s.total_q)
    _say(f"[gpu] full-size {case.name}: rows {s.total_q}, context {case.batch.max_seq_len}, "
         f"sampled rows {rows}")
    lat_np, own_sets = {}, {}
    for d in case.layers:
        l = d["layer"]
        li = case.inputs[l]
        run.run_layer_split(l)
        torch.cuda.synchronize()
        assert run.fault_bits() == 0
        if d["topk_source_layer"] < 0:
            got = t_np(run.scores_view()[rows]).astype(np.float64)
            ref = O.indexer_scores(s, t_np(li.idx_pool), case.fmt, t_np(li.q_idx),
                                   t_np(li.q_idx_scale), t_np(li.w_idx), d["idx_ssmax_s"],
                                   run.ld, rows)
            gi_all, gl_all = t_np(run.topk_idx[l]), t_np(run.topk_len[l])
            for i, r in enumerate(rows):
                p = int(s.q_pos[r])
                assert (got[i, p + 1:case.batch.max_seq_len] == -np.inf).all(), (l, r)
                err = np.abs(got[i, :p + 1] - ref[i, :p + 1]).max() / np.abs(ref[i, :p + 1]).max()
                assert err <= SCORE_RTOL, f"layer {l} row {r}: score rel err {err:.3e}"
                oi, on = O.topk_row(got[i], p, d["top_k"])
                assert int(gl_all[r]) == on, (l, r)
                assert np.array_equal(gi_all[r], oi), f"layer {l} row {r}: top-k differs"
            ties, log = check_topk_rows(gi_all, gl_all, ref, s.q_pos, d["top_k"], rows)
            _say(f"  layer {l}: scores and top-k ok (fp64 near-ties {ties})")
            own_sets[l] = [O.topk_row(ref[i], int(s.q_pos[r]), d["top_k"]) for i, r in
                           enumerate(rows)]
        idx, ln = run.topk_of(l)
        gi, gl = t_np(idx), t_np(ln)
        lat_l = d["kv_sharing_target_layer"] if d["kv_sharing_target_layer"] >= 0 else l
        if lat_l not in lat_np:
            lat_np[lat_l] = t_np(case.inputs[lat_l].lat_pool)
        q_bits = t_np(li.q_mla)
        o, lse = O.sparse_mla(s, lat_np[lat_l], case.fmt, q_bits, d["rope_dim"], gi, gl,
                              d["softmax_scale"], d["ssmax_s"], rows=rows)
        go = O.decode_bf16(t_np(run.out[l][rows]))
        gls = t_np(run.lse[l][rows])
        eo = check_close(go, o, f"{case.name} L{l} out")
        el = check_close(gls, lse, f"{case.name} L{l} lse")
        _say(f"  layer {l}: attention max|d| out {eo:.3e} lse {el:.3e}")
        # end to end: attention on the oracle's own selection (the source layer's for a
        # shared-indexer layer)
        src = d["topk_source_layer"] if d["topk_source_layer"] >= 0 else l
        oi_all, ol_all = gi.copy(), gl.copy()
        same = True
        for i, r in enumerate(rows):
            oi, on = own_sets[src][i]
            oi_all[r], ol_all[r] = oi, on
            same &= bool(on == int(gl[r]) and np.array_equal(oi, gi[r]))
        o2, lse2 = O.sparse_mla(s, lat_np[lat_l], case.fmt, q_bits, d["rope_dim"], oi_all,
                                ol_all, d["softmax_scale"], d["ssmax_s"], rows=rows)
        e2o = float(np.abs(go - o2).max())
        e2l = float(np.abs(gls - lse2).max())
        _say(f"  layer {l}: end to end on the oracle's own top-k (sets equal: {same}): "
             f"max|d| out {e2o:.3e} lse {e2l:.3e}")
        if same:
            check_close(go, o2, f"{case.name} L{l} end-to-end out")
            check_close(gls, lse2, f"{case.name} L{l} end-to-end lse")


def test_full_size_second_layouts_sampled_rows():
    """The bench's side measurements at the verify workload's full size (its first layer's
    selections): sparse MLA over a bf16 1,152-B-row cache and over a plain-E4M3 576-B-row
    cache with FP8 queries, and sliding-window MLA over the last 2,048 positions of the
    fp8_ds_mla cache -- the same generators and seeds as the bench -- checked on sampled
    rows against the oracle."""
    case = synth.config(3, device=DEV)
    torch.cuda.synchronize()
    run = CaseRunner(case)
    d = case.layers[0]
    l = d["layer"]
    run.run_layer_split(l)
    torch.cuda.synchronize()
    assert run.fault_bits() == 0
    b = case.batch
    s = batch_np(b)
    rows = _sample_rows(s.total_q)
    H, rope, K = case.mla_heads, d["rope_dim"], d["top_k"]
    li = case.inputs[l]
    nb, bs = li.lat_pool.shape[0], li.lat_pool.shape[1]
    pool16 = synth.make_latent_pool(77, nb, bs, "bf16", device=DEV)
    pool8, kv_scale = synth.make_plain_e4m3_pool(78, nb, bs, device=DEV)
    q8, q8s = synth.make_mla_query_fp8(79, b.total_q, H, rope, device=DEV)
    idx, ln = run.topk_of(l)
    gi, gl = t_np(idx), t_np(ln)
    out = torch.empty((b.total_q, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((b.total_q, H), dtype=torch.float32, device=DEV)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, run.seqs, H, K)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    q_bits = t_np(li.q_mla)
    win_idx, win_len = O.window_positions(s.q_pos, K)
    checks = (
        ("bf16_rows", lambda: M.ml4_sparse_mla_decode(
            run.seqs, M.make_cache(pool16, M.ML4_LAT_BF16_1152), li.q_mla, M.ML4_BF16, H, rope,
            idx, ln, K, d["softmax_scale"], d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault),
         lambda: O.sparse_mla(s, t_np(pool16), "bf16", q_bits, rope, gi, gl,
                              d["softmax_scale"], d["ssmax_s"], rows=rows)),
        ("e4m3_rows", lambda: M.ml4_sparse_mla_decode_e4m3(
            run.seqs, M.make_cache(pool8, M.ML4_LAT_E4M3_576), kv_scale, q8, q8s, H, rope, idx,
            ln, K, d["softmax_scale"], d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault),
         lambda: O.sparse_mla(s, t_np(pool8), "e4m3", t_np(q8), rope, gi, gl,
                              d["softmax_scale"], d["ssmax_s"], rows=rows, q_scale=t_np(q8s),
                              kv_scale=kv_scale)),
        ("window2048_fp8", lambda: M.ml4_window_mla_decode(
            run.seqs, run.lat_caches[l], li.q_mla, M.ML4_BF16, H, rope, K, d["softmax_scale"],
            d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault),
         lambda: O.sparse_mla(s, t_np(li.lat_pool), "fp8", q_bits, rope, win_idx, win_len,
                              d["softmax_scale"], d["ssmax_s"], rows=rows)),
    )
    for name, gpu, oracle in checks:
        gpu()
        torch.cuda.synchronize()
        assert M.ml4_fault_query(fault) == 0, name
        o, ls = oracle()
        eo = check_close(O.decode_bf16(t_np(out[rows])), o, f"{name} out")
        el = check_close(t_np(lse[rows]), ls, f"{name} lse")
        _say(f"  {name}: max|d| out {eo:.3e} lse {el:.3e}")
