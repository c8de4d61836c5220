"""Parity at the five workloads' full sizes, on the inputs and through the entries the bench
times (MI355X only): the seeded workload is generated on the GPU exactly as the bench does
and each layer runs through the separate entries with the bench's launch configuration.
On sampled query rows (first, middle, last) the oracle recomputes, one row at a time:

* indexer scores over every visible key, within 2e-5 of the row's largest |score| (fp32
  accumulation of exact e4m3 products), -inf past the row's position;
* the top-k list, bit-exact against the oracle's exact selection on the kernel's own fp32
  scores (the integer decision taken in the kernel's precision), and against the oracle's
  fp64 scores up to near-ties (tests/compare.py);
* attention output and LSE, |d| <= 2e-3 + 1e-2 |ref|, with the layer modes resolved as the
  bench runs them (shared-indexer layers reuse the owner's top-k, consumers read the
  owner's latent cache).
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
    return sorted({0, total_q // 2, total_q - 1})


@pytest.mark.parametrize("config", [2, 3, 4, 5])
def test_full_size_workload_sampled_rows(config):
    case = synth.config(config, device=DEV)          # the bench's inputs (same seed)
    torch.cuda.synchronize()
    run = CaseRunner(case)
    s = batch_np(case.batch)
    rows = _sample_rows(s.total_q)
    _say(f"[gpu] full-size {case.name}: rows {s.total_q}, context {case.batch.max_seq_len}, "
         f"sampled rows {rows}")
    lat_np = {}
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
        idx, ln = run.topk_of(l)
        gi, gl = t_np(idx), t_np(ln)
        lat_l = d["kv_sharing_target_layer"] if d["kv_sharing_target_layer"] >= 0 else l
        if lat_l not in lat_np:
            lat_np[lat_l] = t_np(case.inputs[lat_l].lat_pool)
        o, lse = O.sparse_mla(s, lat_np[lat_l], case.fmt, t_np(li.q_mla), d["rope_dim"], gi, gl,
                              d["softmax_scale"], d["ssmax_s"], rows=rows)
        go = O.decode_bf16(t_np(run.out[l][rows]))
        eo = check_close(go, o, f"{case.name} L{l} out")
        el = check_close(t_np(run.lse[l][rows]), lse, f"{case.name} L{l} lse")
        _say(f"  layer {l}: attention max|d| out {eo:.3e} lse {el:.3e}")
