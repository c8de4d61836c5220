"""Parity of the HIP path with the CPU oracle on the same seeded inputs (MI355X only).

Every GPU call goes through the C ABI (ctypes binding).  Comparison rules (tests/compare.py):
top-k sets bit-exact up to logged near-ties within 1e-6 of the k-th score; top-k on given
fp32 scores bit-exact; attention |d| <= 2e-3 + 1e-2 |ref|; indexer scores within an fp32
rounding bound.
"""

import math

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
SCORE_RTOL = 2e-5   # fp32 accumulation of exact e4m3 products over 128 dims and <= 64 heads


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _say(msg):
    print(msg, flush=True)


def small_cases():
    """Same recipe as the five workloads, at sizes the oracle finishes in seconds, with
    ragged lengths (not multiples of 16 or 64) and several tiles per work-group."""
    L = synth.layer_desc
    return {
        "c1_fp32_4096": synth.config(1),
        "c2_decode_ragged": synth.make_case(
            "c2r", 21, seq_lens=[2100, 1000, 3333, 65], q_per_seq=[1, 1, 1, 1], block_size=64,
            fmt="fp8", idx_heads=64, mla_heads=128, layers=[L(0, top_k=2048)], extra_blocks=5),
        "c3_verify_rope_nope": synth.make_case(
            "c3s", 31, seq_lens=[4099, 2600, 5000], q_per_seq=[4, 4, 4], block_size=64,
            fmt="fp8", idx_heads=64, mla_heads=128,
            layers=[L(0, ssmax_s=0.3), L(1, rope_dim=0, ssmax_s=0.3)]),
        "c4_modes_3layer": synth.make_case(
            "c4s", 41, seq_lens=[20000], q_per_seq=[1], block_size=64, fmt="fp8",
            idx_heads=64, mla_heads=128,
            layers=[L(0), L(1, topk_source_layer=0), L(2, kv_sharing_target_layer=0)]),
        "c5_prefill_causal": synth.make_case(
            "c5s", 51, seq_lens=[3000], q_per_seq=[300], block_size=64, fmt="fp8",
            idx_heads=64, mla_heads=128, layers=[L(0, top_k=2048)]),
        "r2_verify_ragged": synth.make_case(
            "r2v", 71, seq_lens=[9001, 17000, 3], q_per_seq=[2, 2, 1], block_size=64,
            fmt="fp8", idx_heads=64, mla_heads=128, layers=[L(0, ssmax_s=0.3)]),
        "h48_decode_rows": synth.make_case(
            "h48", 81, seq_lens=[3001, 700, 4500], q_per_seq=[1, 1, 1], block_size=32,
            fmt="fp8", idx_heads=48, mla_heads=32, layers=[L(0, top_k=1024, idx_ssmax_s=0.2)]),
        "h16_decode_rows": synth.make_case(
            "h16d", 83, seq_lens=[2500, 130], q_per_seq=[1, 1], block_size=64,
            fmt="fp8", idx_heads=16, mla_heads=16, layers=[L(0, top_k=512)]),
        "h32_decode_rows": synth.make_case(
            "h32d", 85, seq_lens=[5100], q_per_seq=[1], block_size=16,
            fmt="fp8", idx_heads=32, mla_heads=48, layers=[L(0, top_k=2048)]),
        "h16_h64_blocks16": synth.make_case(
            "hx", 61, seq_lens=[900, 1500], q_per_seq=[2, 1], block_size=16, fmt="fp8",
            idx_heads=32, mla_heads=16, layers=[L(0, top_k=512, idx_ssmax_s=0.25)]),
        # 11, 8 and 2 rows per request: full 4-row indexer groups and groups of 3 and 2, 32
        # indexer heads, 16-token blocks; the last request's rows sit at positions 0 and 1,
        # so with SSMax the attention logit scale of position 0 is zero (one key)
        "r8_rows_h32": synth.make_case(
            "r8", 91, seq_lens=[5000, 2300, 2], q_per_seq=[11, 8, 2], block_size=16,
            fmt="fp8", idx_heads=32, mla_heads=64,
            layers=[L(0, top_k=1024, idx_ssmax_s=0.2, ssmax_s=0.3)]),
    }


CASES = small_cases()


def _oracle_scores(case, s, l, ld, rows=None):
    li = case.inputs[l]
    d = [x for x in case.layers if x["layer"] == l][0]
    return O.indexer_scores(s, t_np(li.idx_pool), case.fmt, t_np(li.q_idx), t_np(li.q_idx_scale),
                            t_np(li.w_idx), d["idx_ssmax_s"], ld, rows)


def _decode_out(case, t):
    return O.decode_bf16(t_np(t)) if case.fmt == "fp8" else t_np(t).astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_step_matches_oracle(name):
    case = CASES[name]
    _say(f"[gpu] layer step {name}")
    dev = synth.case_to(case, DEV)
    run = CaseRunner(dev)
    run.run_step(fused=True)
    torch.cuda.synchronize()
    assert run.fault_bits() == 0
    s = batch_np(case.batch)
    store = {}
    for d in case.layers:
        l = d["layer"]
        li = case.inputs[l]
        if d["topk_source_layer"] < 0:
            ref = _oracle_scores(case, s, l, run.ld)
            gi, gl = t_np(run.topk_idx[l]), t_np(run.topk_len[l])
            ties, log = check_topk_rows(gi, gl, ref, s.q_pos, d["top_k"])
            _say(f"  layer {l}: top-k tie exceptions {ties} {log[:3]}")
            store[l] = (gi, gl)
        gi, gl = store[d["topk_source_layer"]] if d["topk_source_layer"] >= 0 else store[l]
        lat_l = d["kv_sharing_target_layer"] if d["kv_sharing_target_layer"] >= 0 else l
        o, lse = O.sparse_mla(s, t_np(case.inputs[lat_l].lat_pool), case.fmt, t_np(li.q_mla),
                              d["rope_dim"], gi, gl, d["softmax_scale"], d["ssmax_s"])
        eo = check_close(_decode_out(case, run.out[l]), o, f"{name} L{l} out")
        el = check_close(t_np(run.lse[l]), lse, f"{name} L{l} lse")
        _say(f"  layer {l}: max|d| out {eo:.3e} lse {el:.3e}")


@pytest.mark.parametrize("name", ["c1_fp32_4096", "c2_decode_ragged", "c3_verify_rope_nope",
                                  "c5_prefill_causal", "r2_verify_ragged", "h48_decode_rows",
                                  "h16_decode_rows", "h32_decode_rows", "h16_h64_blocks16",
                                  "r8_rows_h32"])
def test_indexer_scores_match_oracle(name):
    case = CASES[name]
    _say(f"[gpu] indexer {name}")
    dev = synth.case_to(case, DEV)
    run = CaseRunner(dev)
    l = case.layers[0]["layer"]
    li = dev.inputs[l]
    L = run.desc[l]
    sc = torch.full((case.batch.total_q, run.ld), 12345.0, device=DEV)
    M.ml4_indexer_score(run.seqs, run.idx_caches[l], li.q_idx, run.qi_dtype, li.q_idx_scale,
                        li.w_idx, L.idx_heads, L.idx_ssmax_s, sc, run.ld, run.fault)
    torch.cuda.synchronize()
    assert run.fault_bits() == 0
    s = batch_np(case.batch)
    ref = _oracle_scores(case, s, l, run.ld)
    got = t_np(sc).astype(np.float64)
    maxlen = case.batch.max_seq_len
    for r in range(s.total_q):
        p = int(s.q_pos[r])
        assert (got[r, p + 1:maxlen] == -np.inf).all(), f"row {r}: tail not -inf"
        g, f = got[r, :p + 1], ref[r, :p + 1]
        scale = np.abs(f).max()
        err = np.abs(g - f) / max(scale, 1e-30)
        assert err.max() <= SCORE_RTOL, f"row {r}: rel err {err.max():.3e}"
    rel = np.max([np.max(np.abs(got[r, :int(s.q_pos[r]) + 1] - ref[r, :int(s.q_pos[r]) + 1]) /
                         max(np.abs(ref[r, :int(s.q_pos[r]) + 1]).max(), 1e-30))
                  for r in range(s.total_q)])
    _say(f"  max error relative to row max: {rel:.3e}")


def _rand_scores(n, seed, dup_levels=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, generator=g)
    if dup_levels:
        x = torch.round(x * dup_levels) / dup_levels      # many exact ties
    return x


@pytest.mark.parametrize("n,top_k,seed", [(100, 256, 1), (5000, 2048, 2), (32768, 2048, 3),
                                          (32769, 2048, 4), (70000, 2048, 5), (131072, 1, 6),
                                          (140000, 2048, 7), (300001, 777, 8)])
def test_topk_exact_on_given_scores(n, top_k, seed):
    """Integer selection: identical index sets and lengths to the oracle on the same fp32
    scores, including heavy ties, signed zeros, -inf and a NaN (which raises the fault bit)."""
    _say(f"[gpu] topk n={n} k={top_k}")
    rows = []
    for i in range(3):
        x = _rand_scores(n, seed * 10 + i, dup_levels=[None, 8, 2][i])
        if i == 2:
            x[::7] = 0.0
            x[1::7] = -0.0
            x[3::11] = -math.inf
        rows.append(x)
    has_nan = n > top_k         # rows with n <= k are returned whole, scores unread
    if has_nan:
        rows[1][n // 3] = math.nan
    ld = (n + 3) // 4 * 4
    scores = torch.full((3, ld), -5.0)
    for i, x in enumerate(rows):
        scores[i, :n] = x
    batch = synth.make_batch(seed, [n, n, n], [1, 1, 1], 64, device=DEV)
    seqs = M.make_seqs(batch)
    idx = torch.full((3, top_k), -9, dtype=torch.int32, device=DEV)
    ln = torch.zeros(3, dtype=torch.int32, device=DEV)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, top_k)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    sd = scores.to(DEV)
    M.ml4_topk_select(seqs, sd, ld, top_k, idx, ln, ws, wsn, fault)
    torch.cuda.synchronize()
    bits = M.ml4_fault_query(fault)
    assert bits == (M.ML4_FAULT_NAN_SCORE if has_nan else 0)
    gi, gl = t_np(idx), t_np(ln)
    sn = scores.numpy().astype(np.float64)
    for r in range(3):
        oi, on = O.topk_row(sn[r], n - 1, top_k)
        assert gl[r] == on
        assert np.array_equal(gi[r], oi), f"row {r}: first diff at {np.argmax(gi[r] != oi)}"


def test_topk_long_rows_of_mixed_lengths():
    """The multi-work-group selection (rows above 131,072 positions) with rows of unequal
    length in one launch: a row shorter than k (returned whole), one in the one-work-group
    range, long rows whose chunk counts differ (so some work-groups of the grid have no
    keys of their row) and a row of 2,500 positions (fewer than the long-row sample's rank
    would ask for); every row equals the oracle's, and a second call on the same workspace
    gives the same result."""
    lens = [140000, 1500, 200003, 70000, 131073, 2500]
    top_k = 2048
    _say(f"[gpu] topk mixed long rows {lens} k={top_k}")
    n_max = max(lens)
    ld = (n_max + 3) // 4 * 4
    scores = torch.full((len(lens), ld), -5.0)
    for i, n in enumerate(lens):
        x = _rand_scores(n, 900 + i, dup_levels=[None, 4, 16, None, 2, None][i])
        scores[i, :n] = x
    batch = synth.make_batch(77, lens, [1] * len(lens), 64, device=DEV)
    seqs = M.make_seqs(batch)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, top_k)
    assert wsn > 0
    ws = torch.empty(wsn, dtype=torch.uint8, device=DEV)
    sd = scores.to(DEV)
    sn = scores.numpy().astype(np.float64)
    pos = t_np(batch.q_pos)
    for call in range(2):
        idx = torch.full((len(lens), top_k), -9, dtype=torch.int32, device=DEV)
        ln = torch.zeros(len(lens), dtype=torch.int32, device=DEV)
        fault = torch.zeros(1, dtype=torch.int32, device=DEV)
        M.ml4_topk_select(seqs, sd, ld, top_k, idx, ln, ws, wsn, fault)
        torch.cuda.synchronize()
        assert M.ml4_fault_query(fault) == 0
        gi, gl = t_np(idx), t_np(ln)
        for r in range(len(lens)):
            oi, on = O.topk_row(sn[r], int(pos[r]), top_k)
            assert gl[r] == on, (call, r)
            assert np.array_equal(gi[r], oi), f"call {call} row {r}: first diff at {np.argmax(gi[r] != oi)}"


def test_topk_rows_of_millions_of_positions():
    """Rows of 3,000,001 and 6,500,000 positions in one launch (the long-row filter's sample
    grows with the row: 16,384 and 32,768 keys), one of them with many ties: the selected
    sets equal the oracle's."""
    lens = [3000001, 6500000]
    top_k = 2048
    _say(f"[gpu] topk rows of millions {lens} k={top_k}")
    ld = (max(lens) + 3) // 4 * 4
    scores = torch.full((len(lens), ld), -5.0)
    for i, n in enumerate(lens):
        scores[i, :n] = _rand_scores(n, 4100 + i, dup_levels=[None, 64][i])
    batch = synth.make_batch(78, lens, [1] * len(lens), 64, device=DEV)
    seqs = M.make_seqs(batch)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, top_k)
    ws = torch.empty(wsn, dtype=torch.uint8, device=DEV)
    idx = torch.full((len(lens), top_k), -9, dtype=torch.int32, device=DEV)
    ln = torch.zeros(len(lens), dtype=torch.int32, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_topk_select(seqs, scores.to(DEV), ld, top_k, idx, ln, ws, wsn, fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    gi, gl = t_np(idx), t_np(ln)
    pos = t_np(batch.q_pos)
    for r in range(len(lens)):
        oi, on = O.topk_row(scores[r].numpy().astype(np.float64), int(pos[r]), top_k)
        assert gl[r] == on
        assert np.array_equal(gi[r], oi), f"row {r}: first diff at {np.argmax(gi[r] != oi)}"


@pytest.mark.parametrize("n,top_k,kind", [(20000, 2048, "const"), (50000, 2048, "tie_block"),
                                          (9000, 2048, "const"), (200000, 2048, "const"),
                                          (300000, 2048, "tie_block"),
                                          (300000, 2048, "tie_block_20k")])
def test_topk_when_the_candidate_list_overflows(n, top_k, kind):
    """Rows whose keys above the sampled threshold do not fit the candidate list (massive
    ties at the threshold) take the streaming selection; the result is still the oracle's.
    On long rows 9,000 tied keys fit the list (ties resolved in it, lowest positions
    first) and 20,000 do not."""
    _say(f"[gpu] topk overflow n={n} k={top_k} {kind}")
    g = torch.Generator().manual_seed(n)
    if kind == "const":
        x = torch.full((n,), 0.25)
    else:
        x = torch.clamp(torch.randn(n, generator=g), max=2.9)
        x[torch.randperm(n, generator=g)[:20000 if kind == "tie_block_20k" else 9000]] = 3.0
    ld = (n + 3) // 4 * 4
    scores = torch.full((1, ld), -5.0)
    scores[0, :n] = x
    batch = synth.make_batch(1, [n], [1], 64, device=DEV)
    seqs = M.make_seqs(batch)
    idx = torch.full((1, top_k), -9, dtype=torch.int32, device=DEV)
    ln = torch.zeros(1, dtype=torch.int32, device=DEV)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, top_k)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_topk_select(seqs, scores.to(DEV), ld, top_k, idx, ln, ws, wsn, fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    oi, on = O.topk_row(scores.numpy()[0].astype(np.float64), n - 1, top_k)
    assert t_np(ln)[0] == on
    assert np.array_equal(t_np(idx)[0], oi)


def test_topk_long_row_whose_sample_overestimates_the_threshold():
    """A long row built so that the threshold taken from its sample keeps fewer than k keys:
    the row's sample slots (2,048 float4 vectors at (j * n4) // 2,048, j < 2,048; white-box
    knowledge of the long-row filter) start with a large key, one of them is left out, so
    2,047 keys lie above every other key and the sample's rank-k-scaled key is one of them.
    The selection must notice the short list and fall back; the result is the oracle's."""
    n, top_k = 300000, 2048
    _say(f"[gpu] topk long-row sample miss n={n} k={top_k}")
    g = torch.Generator().manual_seed(5)
    x = torch.randn(n, generator=g)
    n4 = (n + 3) // 4
    slots = torch.tensor([4 * ((j * n4) // 2048) for j in range(1, 2048)])
    x[slots] = 10.0
    ld = (n + 3) // 4 * 4
    scores = torch.full((1, ld), -5.0)
    scores[0, :n] = x
    batch = synth.make_batch(2, [n], [1], 64, device=DEV)
    seqs = M.make_seqs(batch)
    idx = torch.full((1, top_k), -9, dtype=torch.int32, device=DEV)
    ln = torch.zeros(1, dtype=torch.int32, device=DEV)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, top_k)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_topk_select(seqs, scores.to(DEV), ld, top_k, idx, ln, ws, wsn, fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    oi, on = O.topk_row(scores.numpy()[0].astype(np.float64), n - 1, top_k)
    assert t_np(ln)[0] == on
    assert np.array_equal(t_np(idx)[0], oi)
    assert set(slots.tolist()) <= set(t_np(idx)[0].tolist())


def _topk_lists(case, seed, top_k):
    """Seeded selections: distinct ascending positions in [0, p] per row, ragged lengths."""
    g = np.random.default_rng(seed)
    q_pos = case.batch.q_pos.cpu().numpy()
    idx = np.full((len(q_pos), top_k), -1, dtype=np.int32)
    ln = np.zeros(len(q_pos), dtype=np.int32)
    for r, p in enumerate(q_pos):
        n = min(top_k, int(p) + 1)
        if r % 3 == 1:
            n = max(1, n // 3)          # short selections (top-k compaction)
        sel = np.sort(g.choice(int(p) + 1, size=n, replace=False))
        idx[r, :n] = sel
        ln[r] = n
    return idx, ln


@pytest.mark.parametrize("name,heads", [("c2_decode_ragged", 128), ("c3_verify_rope_nope", 128),
                                        ("h16_h64_blocks16", 16), ("c1_fp32_4096", 16),
                                        ("c2_decode_ragged", 64)])
def test_sparse_mla_matches_oracle(name, heads):
    case = CASES[name]
    _say(f"[gpu] mla {name} H={heads}")
    dev = synth.case_to(case, DEV)
    run = CaseRunner(dev)
    s = batch_np(case.batch)
    for d in case.layers:
        l = d["layer"]
        if case.inputs[l].lat_pool is None:
            continue
        idx, ln = _topk_lists(case, 100 + l, d["top_k"])
        q = dev.inputs[l].q_mla[:, :heads].contiguous()
        out = torch.empty((s.total_q, heads, 512), dtype=run.out[l].dtype, device=DEV)
        lse = torch.empty((s.total_q, heads), dtype=torch.float32, device=DEV)
        wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, run.seqs, heads, d["top_k"])
        ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
        M.ml4_sparse_mla_decode(run.seqs, run.lat_caches[l], q, run.qm_dtype, heads,
                                d["rope_dim"], torch.from_numpy(idx).to(DEV),
                                torch.from_numpy(ln).to(DEV), d["top_k"], d["softmax_scale"],
                                d["ssmax_s"], out, run.qm_dtype, lse, ws, wsn, run.fault)
        torch.cuda.synchronize()
        assert run.fault_bits() == 0
        o, l_ref = O.sparse_mla(s, t_np(case.inputs[l].lat_pool), case.fmt, t_np(q.cpu()),
                                d["rope_dim"], idx, ln, d["softmax_scale"], d["ssmax_s"])
        eo = check_close(_decode_out(case, out), o, "out")
        el = check_close(t_np(lse), l_ref, "lse")
        _say(f"  layer {l} (rope {d['rope_dim']}, splits {wsn > 0}): max|d| {eo:.3e} {el:.3e}")


def test_modes_are_bit_identical_to_their_definitions():
    """Shared-indexer layer == MLA on the source's top-k; consumer layer == MLA on the
    owner's cache; fused == separate entries; repeated runs identical (no races)."""
    case = CASES["c4_modes_3layer"]
    dev = synth.case_to(case, DEV)
    run = CaseRunner(dev)
    run.run_step(fused=True)
    torch.cuda.synchronize()
    outs = {l: run.out[l].clone() for l in run.out}
    idx0, len0 = run.topk_idx[0].clone(), run.topk_len[0].clone()
    # shared-indexer L1: reads L0's top-k, its own latent cache
    d1 = run.desc[1]
    o1 = torch.empty_like(run.out[1])
    M.ml4_sparse_mla_decode(run.seqs, run.lat_caches[1], dev.inputs[1].q_mla, run.qm_dtype,
                            d1.mla_heads, d1.rope_dim, idx0, len0, d1.top_k, d1.softmax_scale,
                            d1.ssmax_s, o1, run.qm_dtype, None, run.ws, run.ws_bytes, run.fault)
    # consumer L2: its own top-k, L0's latent cache
    d2 = run.desc[2]
    o2 = torch.empty_like(run.out[2])
    M.ml4_sparse_mla_decode(run.seqs, run.lat_caches[0], dev.inputs[2].q_mla, run.qm_dtype,
                            d2.mla_heads, d2.rope_dim, run.topk_idx[2], run.topk_len[2], d2.top_k,
                            d2.softmax_scale, d2.ssmax_s, o2, run.qm_dtype, None, run.ws,
                            run.ws_bytes, run.fault)
    torch.cuda.synchronize()
    assert torch.equal(o1, outs[1]) and torch.equal(o2, outs[2])
    # separate entries and a second run reproduce every output bit for bit
    run.run_step(fused=False)
    torch.cuda.synchronize()
    for l in outs:
        assert torch.equal(run.out[l], outs[l]), f"layer {l} not reproducible"
    assert torch.equal(run.topk_idx[0], idx0)
    assert run.fault_bits() == 0


def test_block_table_permutation_and_nope_rope_bytes():
    case = CASES["c3_verify_rope_nope"]
    dev = synth.case_to(case, DEV)
    run = CaseRunner(dev)
    run.run_step()
    torch.cuda.synchronize()
    base = {l: (run.out[l].clone(), run.topk_idx[l].clone()) for l in run.out}
    # move every physical block and rewrite the table accordingly
    nb = case.batch.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(5)).to(torch.int32)
    case2 = synth.case_to(case, "cpu")
    case2.batch = synth.Batch(case.batch.seq_lens, case.batch.q_start, case.batch.q_pos,
                              perm[case.batch.block_table.long()].contiguous(),
                              case.batch.block_size, nb, case.batch.max_seq_len,
                              case.batch.max_q_per_seq)
    inv = torch.empty_like(perm)
    inv[perm.long()] = torch.arange(nb, dtype=torch.int32)
    for l, li in case2.inputs.items():
        li.idx_pool = li.idx_pool[inv.long()].contiguous()
        li.lat_pool = li.lat_pool[inv.long()].contiguous()
    # the NoPE layer's RoPE bytes hold NaN already; overwrite them with other garbage too
    case2.inputs[1].lat_pool[..., 528:] = 0x7F
    dev2 = synth.case_to(case2, DEV)
    run2 = CaseRunner(dev2)
    run2.run_step()
    torch.cuda.synchronize()
    for l in base:
        assert torch.equal(run2.topk_idx[l], base[l][1])
        assert torch.equal(run2.out[l], base[l][0]), f"layer {l}"
    assert torch.isfinite(run2.out[1].float()).all()


def test_device_faults_are_reported_and_contained():
    case = CASES["c2_decode_ragged"]
    bad = synth.case_to(case, "cpu")
    bt = bad.batch.block_table.clone()
    bt[1, 3] = 1 << 30                   # request 1: a block id outside the pool
    bad.batch = synth.Batch(bad.batch.seq_lens, bad.batch.q_start, bad.batch.q_pos, bt,
                            bad.batch.block_size, bad.batch.num_blocks, bad.batch.max_seq_len,
                            bad.batch.max_q_per_seq)
    dev = synth.case_to(bad, DEV)
    run = CaseRunner(dev)
    run.run_step()
    torch.cuda.synchronize()
    assert run.fault_bits() & M.ML4_FAULT_BLOCK_ID
    # other requests are unaffected: their top-k matches the clean run
    ok = CaseRunner(synth.case_to(case, DEV))
    ok.run_step()
    torch.cuda.synchronize()
    for r in (0, 2, 3):
        assert torch.equal(run.topk_idx[0][r], ok.topk_idx[0][r])
        assert torch.equal(run.out[0][r], ok.out[0][r])
    # an out-of-range top-k entry
    idx = ok.topk_idx[0].clone()
    idx[0, 0] = 10 ** 6
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    d = ok.desc[0]
    M.ml4_sparse_mla_decode(ok.seqs, ok.lat_caches[0], ok.case.inputs[0].q_mla, ok.qm_dtype,
                            d.mla_heads, d.rope_dim, idx, ok.topk_len[0], d.top_k,
                            d.softmax_scale, d.ssmax_s, torch.empty_like(ok.out[0]), ok.qm_dtype,
                            None, ok.ws, ok.ws_bytes, fault)
    assert M.ml4_fault_query(fault) == M.ML4_FAULT_TOPK_INDEX
    # a bit already set by the host is reported as is
    fault.fill_(-(1 << 31))              # bit 31, as an int32
    assert M.ml4_fault_query(fault) == 1 << 31


def test_fp8_ds_mla_range_fault_is_reported_and_contained():
    """A non-finite bf16 query element (row 1) and a selected key whose latent scale exceeds
    128 (one of row 2's keys; P * scale must stay in fp16) each raise ML4_FAULT_RANGE; rows
    that touch neither are bit-identical to the clean run."""
    case = CASES["c2_decode_ragged"]
    _say("[gpu] fp8_ds_mla range fault: query element inf in row 1, key scale 200 in row 2")
    d = case.layers[0]
    idx, ln = _topk_lists(case, 300, d["top_k"])
    s = batch_np(case.batch)

    def run_mla(c):
        dev = synth.case_to(c, DEV)
        run = CaseRunner(dev)
        out = torch.empty_like(run.out[0])
        lse = torch.empty_like(run.lse[0])
        fault = torch.zeros(1, dtype=torch.int32, device=DEV)
        M.ml4_sparse_mla_decode(run.seqs, run.lat_caches[0], dev.inputs[0].q_mla, run.qm_dtype,
                                case.mla_heads, d["rope_dim"], torch.from_numpy(idx).to(DEV),
                                torch.from_numpy(ln).to(DEV), d["top_k"], d["softmax_scale"],
                                d["ssmax_s"], out, run.qm_dtype, lse, run.ws, run.ws_bytes,
                                fault)
        torch.cuda.synchronize()
        return out.cpu(), lse.cpu(), M.ml4_fault_query(fault)

    o0, l0, f0 = run_mla(case)
    assert f0 == 0
    bad = synth.case_to(case, "cpu")
    q = bad.inputs[0].q_mla.clone()
    q[1, 5, 100] = float("inf")
    pool = bad.inputs[0].lat_pool.clone()
    t = int(idx[2, ln[2] // 2])                  # a key row 2 selects
    b2 = int(np.searchsorted(s.q_start, 2, side="right") - 1)
    blk, off = int(s.block_table[b2, t // s.block_size]), t % s.block_size
    pool[blk, off, 512 + 4:512 + 8] = torch.tensor([200.0], dtype=torch.float32).view(torch.uint8)
    bad.inputs[0].q_mla, bad.inputs[0].lat_pool = q, pool
    clean_rows = []
    for r in range(s.total_q):
        if r in (1, 2):
            continue
        b = int(np.searchsorted(s.q_start, r, side="right") - 1)
        slots = {int(s.block_table[b, int(p) // s.block_size]) * s.block_size
                 + int(p) % s.block_size for p in idx[r, :ln[r]]}
        assert blk * s.block_size + off not in slots
        clean_rows.append(r)
    o1, l1, f1 = run_mla(bad)
    assert f1 == M.ML4_FAULT_RANGE
    assert clean_rows
    for r in clean_rows:
        assert torch.equal(o1[r], o0[r]) and torch.equal(l1[r], l0[r]), f"row {r} changed"


def test_fp8_ds_mla_query_beyond_fp16_range_matches_oracle():
    """The bf16 query is taken as given: a head whose query elements exceed the fp16 range
    (row 0, head 3, times 2^15: up to ~1e5) matches the oracle and raises nothing."""
    case = CASES["c2_decode_ragged"]
    d = case.layers[0]
    _say("[gpu] fp8_ds_mla query beyond fp16 range")
    big = synth.case_to(case, "cpu")
    q = big.inputs[0].q_mla.clone()
    q[0, 3] = q[0, 3] * 32768.0                  # exact in bf16 (a power of two)
    assert float(q[0, 3].float().abs().max()) > 65504.0
    big.inputs[0].q_mla = q
    idx, ln = _topk_lists(case, 301, d["top_k"])
    dev = synth.case_to(big, DEV)
    run = CaseRunner(dev)
    s = batch_np(case.batch)
    out = torch.empty_like(run.out[0])
    lse = torch.empty_like(run.lse[0])
    M.ml4_sparse_mla_decode(run.seqs, run.lat_caches[0], dev.inputs[0].q_mla, run.qm_dtype,
                            case.mla_heads, d["rope_dim"], torch.from_numpy(idx).to(DEV),
                            torch.from_numpy(ln).to(DEV), d["top_k"], d["softmax_scale"],
                            d["ssmax_s"], out, run.qm_dtype, lse, run.ws, run.ws_bytes, run.fault)
    torch.cuda.synchronize()
    assert run.fault_bits() == 0
    o, l_ref = O.sparse_mla(s, t_np(big.inputs[0].lat_pool), "fp8", t_np(q), d["rope_dim"], idx,
                            ln, d["softmax_scale"], d["ssmax_s"])
    eo = check_close(_decode_out(case, out), o, "out")
    el = check_close(t_np(lse), l_ref, "lse")
    _say(f"  max|d| out {eo:.3e} lse {el:.3e}")
