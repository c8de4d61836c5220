"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test checks the oracle against something other than itself: a library
decoder, closed forms worked by hand, invariances, exhaustive enumeration on tiny
inputs, or an independent library attention routine.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from tests import packing as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def seqs1(block_table, q_pos, block_size, seq_lens=None, q_start=None):
    bt = np.asarray(block_table, dtype=np.int64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if seq_lens is None:
        seq_lens = [int(q_pos.max()) + 1]
    if q_start is None:
        q_start = [0, len(q_pos)]
    return O.Seqs(np.asarray(seq_lens), np.asarray(q_start), q_pos, bt, block_size)


# ----------------------------------------------------------------------------- formats
def test_e4m3_table_matches_torch_ocp_decoder():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    assert O.e4m3_value(0x38) == 1.0 and O.e4m3_value(0x7E) == 448.0
    assert O.e4m3_value(0x01) == 2.0 ** -9 and O.e4m3_value(0x08) == 2.0 ** -6
    assert O.e4m3_value(0xFE) == -448.0


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = O.decode_bf16(bits)
    ok = np.isnan(ref) == np.isnan(mine)
    assert ok.all()
    assert np.array_equal(mine[~np.isnan(ref)], ref[~np.isnan(ref)])


def test_row_and_token_byte_counts_match_pages():
    # per-row sizes: 656 B fp8_ds_mla, 576 B plain E4M3, 1,152 B bf16, 132 B indexer row
    assert O.LAT_ROW_FP8 == 656 and O.LAT_ROW_PLAIN_FP8 == 576 and O.LAT_ROW_BF16 == 1152
    assert O.IDX_ROW_FP8 == 132
    # 72 layers; every 4th NoPE; NoPE layers 39..71 read layer 35; 28 indexer sharers
    nope = O.nope_layers()
    assert len(nope) == 18 and nope[0] == 3 and nope[-1] == 71 and 35 in nope
    assert set(O.KV_CONSUMERS) <= set(nope) and len(O.KV_CONSUMERS) == 9
    owners = O.N_LAYERS - len(O.KV_CONSUMERS)
    indexers = O.N_LAYERS - O.N_INDEX_SHARERS
    assert owners == 63 and indexers == 44
    assert owners * O.LAT_ROW_FP8 == 41328 and indexers * O.IDX_ROW_FP8 == 5808
    assert O.kv_bytes_per_token(O.LAT_ROW_FP8) == 47136
    assert O.kv_bytes_per_token(O.LAT_ROW_PLAIN_FP8) == 42096
    assert O.kv_bytes_per_token(O.LAT_ROW_BF16) == 78384
    assert round(78384 / 42096, 2) == 1.86           # "1.86x the KV capacity of bf16"
    assert round(100 * (72 / 63 - 1), 1) == 14.3      # KV-share dedup gain on HiSparse


# ----------------------------------------------------------------------------- indexer
def _golden_indexer():
    g = json.load(open(os.path.join(GOLDEN, "indexer_handworked.json")))
    pool = P.index_pool(g["num_blocks"], g["block_size"])
    for k in g["keys"]:
        P.put_index_row(pool, k["slot"], k["codes"], k["scale"])
    q = np.zeros((1, 2, 128), dtype=np.uint8)
    for h, cd in g["q_codes"].items():
        for d, c in cd.items():
            q[0, int(h), int(d)] = int(c, 16)
    s = seqs1(g["block_table"], g["q_pos"], g["block_size"])
    return g, pool, q, s


def test_indexer_handworked_example():
    g, pool, q, s = _golden_indexer()
    qs = np.array([g["q_scale"]])
    w = np.array([g["w"]])
    sc = O.indexer_scores(s, pool, "fp8", q, qs, w, 0.0, ld=4)
    assert sc[0, :3].tolist() == g["expected_scores"]
    assert sc[0, 3] == -np.inf
    idx, ln = O.topk_select(sc, s.q_pos, 2)
    assert idx[0].tolist() == g["expected_top2"] and ln[0] == 2
    idx, ln = O.topk_select(sc, s.q_pos, 1)
    assert idx[0].tolist() == g["expected_top1"] and ln[0] == 1
    # the indexer's own SSMax multiplies every score by s * ln(p + 1)
    sc2 = O.indexer_scores(s, pool, "fp8", q, qs, w, 0.5, ld=4)
    m = 0.5 * math.log(3)
    assert np.allclose(sc2[0, :3], m * np.array(g["expected_scores"]), rtol=1e-15, atol=0)


def test_indexer_negative_weight_keeps_relu_inside():
    """w * ReLU(dot), not ReLU(w * dot): a negative head weight must subtract when the
    dot product is positive and contribute nothing when it is negative."""
    g, pool, q, s = _golden_indexer()
    qs = np.array([[1.0, 1.0]])
    w = np.array([[-1.0, 0.0]])
    sc = O.indexer_scores(s, pool, "fp8", q, qs, w, 0.0, ld=3)
    # head0 dots: t0 = 3 (ks 1), t1 = -1 (ks .5), t2 = 1.5 (ks 4)
    assert sc[0].tolist() == [-3.0, 0.0, -6.0]


def test_indexer_one_hot_orientation_rows_and_paging():
    """Head h queries dim h only; key t carries value v_t on dim t % 3.  Then
    score(r, t) = w[r, t%3] * qs[r, t%3] * ReLU(v_t) * ks[t]: catches head/dim swaps,
    row mix-ups between requests and slot-addressing mistakes."""
    H, bs = 3, 4
    rng = np.random.default_rng(3)
    vals = [0x38, 0x40, 0xB8, 0x3C, 0xC0, 0x30, 0x44, 0xB0]     # 1,2,-1,1.5,-2,.5,3,-.5
    n = [7, 5]
    nblocks = 4
    bt = np.array([[3, 0], [2, 1]])
    pool = P.index_pool(nblocks, bs)
    truth = {}
    for b in range(2):
        for t in range(n[b]):
            code = vals[rng.integers(len(vals))]
            ks = float(rng.choice([0.5, 1.0, 2.0]))
            slot = bt[b][t // bs] * bs + t % bs
            P.put_index_row(pool, slot, {t % 3: code}, ks)
            truth[(b, t)] = (O.e4m3_value(code), ks)
    q = np.zeros((2, H, 128), dtype=np.uint8)
    for r in range(2):
        for h in range(H):
            q[r, h, h] = 0x38
    qs = np.array([[1.0, 2.0, 4.0], [0.5, 1.0, 1.0]])
    w = np.array([[1.0, 0.5, 0.25], [2.0, 4.0, 8.0]])
    s = O.Seqs(np.array(n), np.array([0, 1, 2]), np.array([n[0] - 1, n[1] - 1]), bt, bs)
    sc = O.indexer_scores(s, pool, "fp8", q, qs, w, 0.0, ld=8)
    for r in range(2):
        for t in range(8):
            if t >= n[r]:
                assert sc[r, t] == -np.inf
                continue
            v, ks = truth[(r, t)]
            h = t % 3
            assert sc[r, t] == w[r, h] * qs[r, h] * max(v, 0.0) * ks


def test_indexer_homogeneity_and_causal_rows():
    rng = np.random.default_rng(7)
    bs, nb = 16, 6
    pool = rng.integers(0, 256, size=(nb, bs, 132), dtype=np.uint8)
    pool[:, :, :128][pool[:, :, :128] & 0x7F == 0x7F] = 0x11     # no NaN codes
    pool.reshape(-1, 132)[:, 128:] = np.frombuffer(
        rng.uniform(0.5, 2, size=nb * bs).astype("<f4").tobytes(), np.uint8).reshape(-1, 4)
    q = rng.integers(0, 256, size=(4, 5, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x22
    qs = rng.uniform(0.1, 1, size=(4, 5))
    w = rng.uniform(0, 1, size=(4, 5))
    bt = np.array([[5, 1, 3, 0, 2, 4]])
    s = O.Seqs(np.array([90]), np.array([0, 4]), np.array([86, 87, 88, 89]), bt, bs)
    base = O.indexer_scores(s, pool, "fp8", q, qs, w, 0.0, ld=96)
    for r in range(4):
        p = 86 + r
        assert np.isfinite(base[r, :p + 1]).all() and (base[r, p + 1:] == -np.inf).all()
    assert np.allclose(O.indexer_scores(s, pool, "fp8", q, qs, 2 * w, 0.0, 96)[:, :87],
                       2 * base[:, :87], rtol=1e-14)
    assert np.allclose(O.indexer_scores(s, pool, "fp8", q, 3 * qs, w, 0.0, 96)[:, :87],
                       3 * base[:, :87], rtol=1e-14)
    # a block-table permutation with the rows moved alongside changes nothing
    perm = np.array([2, 4, 0, 5, 1, 3])
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    s2 = O.Seqs(s.seq_lens, s.q_start, s.q_pos, perm[bt], bs)
    assert np.array_equal(O.indexer_scores(s2, pool2, "fp8", q, qs, w, 0.0, 96), base)


# ----------------------------------------------------------------------------- top-k
def _dominates(a, b, s):
    """Total order of the selection: higher score first, then lower position; NaN last."""
    sa, sb = s[a], s[b]
    if math.isnan(sa) or math.isnan(sb):
        if math.isnan(sa) and math.isnan(sb):
            return a < b
        return not math.isnan(sa)
    if sa != sb:
        return sa > sb
    return a < b


@pytest.mark.parametrize("seed", range(40))
def test_topk_equals_exhaustive_subset_search(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    vals = rng.integers(-3, 4, size=n).astype(np.float64)        # many duplicates
    if seed % 5 == 0:
        vals[rng.integers(n)] = np.nan
    if seed % 7 == 0:
        vals[rng.integers(n)] = -0.0
    k = int(rng.integers(1, n + 3))
    kk = min(k, n)
    winners = [S for S in itertools.combinations(range(n), kk)
               if all(_dominates(a, b, vals) for a in S for b in range(n) if b not in S)]
    assert len(winners) == 1
    idx, ln = O.topk_row(vals, n - 1, k)
    assert ln == kk
    assert idx[:kk].tolist() == list(winners[0])
    assert (idx[kk:] == -1).all()


def test_topk_special_cases():
    rng = np.random.default_rng(1)
    s = rng.normal(size=50)
    idx, ln = O.topk_row(s, 49, 64)                 # k >= n: everything, ascending
    assert ln == 50 and idx[:50].tolist() == list(range(50)) and (idx[50:] == -1).all()
    s2 = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    idx, ln = O.topk_row(s2, 4, 1)                  # k = 1: first argmax
    assert idx.tolist() == [int(np.argmax(s2))] == [1]
    idx, ln = O.topk_row(s2, 2, 8)                  # masked tail: only 0..p
    assert ln == 3 and idx[:3].tolist() == [0, 1, 2]
    z = np.array([0.0, -0.0, 0.0, -0.0])           # signed zeros are equal: lowest t wins
    assert O.topk_row(z, 3, 2)[0].tolist() == [0, 1]
    e = np.array([np.nan, -np.inf, np.nan, 5.0])     # NaN ranks below -inf
    assert O.topk_row(e, 3, 2)[0].tolist() == [1, 3]
    assert O.topk_row(e, 3, 3)[0].tolist() == [0, 1, 3]
    big = rng.normal(size=2000)
    a = O.topk_row(big, 1999, 300)[0]
    assert np.array_equal(a, O.topk_row(big * 7.5, 1999, 300)[0])   # positive scaling


# ----------------------------------------------------------------------------- sparse MLA
def _one_request(nkeys, bs=8, nb=None, rope_dim=64):
    nb = nb or (nkeys + bs - 1) // bs
    bt = np.arange(nb)[::-1].reshape(1, -1).copy()    # reversed physical order
    return O.Seqs(np.array([nkeys]), np.array([0, 1]), np.array([nkeys - 1]), bt, bs), nb


def test_mla_handworked_two_keys_with_group_scales_and_rope():
    s, nb = _one_request(2, bs=2)
    pool = P.latent_pool(nb, 2)
    slotA, slotB = O.slots(s, 0, np.array([0, 1]))
    rA = np.zeros(64); rA[0] = 1.0
    P.put_latent_row(pool, slotA, {0: 0x38, 130: 0x40}, [1.0, 0.5, 1.0, 1.0], rA)
    P.put_latent_row(pool, slotB, {0: 0xB8}, [2.0, 1.0, 1.0, 1.0])
    qv = np.zeros((1, 1, 576), dtype=np.float32)
    qv[0, 0, 0] = 1.0; qv[0, 0, 130] = 0.5; qv[0, 0, 512] = 0.5
    q = P.bf16_bits(qv)
    o, lse = O.sparse_mla(s, pool, "fp8", q, 64, np.array([[0, 1]]), np.array([2]), 1.0, 0.0)
    # l_A = 1*1 + 0.5*(2*0.5) + 0.5*1 = 2 ; l_B = 1*(-1*2) = -2
    pA = 1.0 / (1.0 + math.exp(-4.0)); pB = 1.0 - pA
    assert math.isclose(o[0, 0, 0], pA * 1.0 + pB * -2.0, rel_tol=1e-14)
    assert math.isclose(o[0, 0, 130], pA * 1.0, rel_tol=1e-14)
    assert np.count_nonzero(o[0, 0]) == 2
    assert math.isclose(lse[0, 0], 2.0 + math.log1p(math.exp(-4.0)), rel_tol=1e-14)
    # NoPE reading of the same rows: the RoPE term drops out, l_A = 1.5
    q0 = P.bf16_bits(qv[:, :, :512])
    o0, lse0 = O.sparse_mla(s, pool, "fp8", q0, 0, np.array([[0, 1]]), np.array([2]), 1.0, 0.0)
    pA0 = 1.0 / (1.0 + math.exp(-3.5))
    assert math.isclose(o0[0, 0, 130], pA0, rel_tol=1e-14)


def _random_latent_case(nkeys, H, rope_dim, seed, bs=8):
    rng = np.random.default_rng(seed)
    s, nb = _one_request(nkeys, bs=bs, rope_dim=rope_dim)
    pool = rng.integers(0, 256, size=(nb, bs, 656), dtype=np.uint8)
    cod = pool[:, :, :512]
    cod[(cod & 0x7F) == 0x7F] = 0x31
    flat = pool.reshape(-1, 656)
    flat[:, 512:528] = np.frombuffer(rng.uniform(0.001, 0.01, size=(nb * bs, 4)).astype("<f4")
                                     .tobytes(), np.uint8).reshape(-1, 16)
    flat[:, 528:656] = np.frombuffer(P.bf16_bits(rng.normal(size=(nb * bs, 64))).astype("<u2")
                                     .tobytes(), np.uint8).reshape(-1, 128)
    q = P.bf16_bits(rng.normal(size=(1, H, 512 + rope_dim)))
    return s, pool, q


def test_mla_single_key_returns_its_row_and_zero_query_gives_mean():
    s, pool, q = _random_latent_case(40, 4, 64, 11)
    c, kr = O.latent_rows_fp8(pool, O.slots(s, 0, np.arange(40)), 64)
    o, lse = O.sparse_mla(s, pool, "fp8", q, 64, np.array([[17] + [-1] * 3]), np.array([1]),
                          0.1, 0.0)
    assert np.array_equal(o[0], np.repeat(c[17][None], 4, axis=0))
    qv = O.decode_bf16(q[0])
    assert np.allclose(lse[0], 0.1 * (qv[:, :512] @ c[17] + qv[:, 512:] @ kr[17]), rtol=1e-13)
    qz = np.zeros_like(q)
    sel = np.array([[3, 5, 8, 13, 21, 34]])
    o, lse = O.sparse_mla(s, pool, "fp8", qz, 64, sel, np.array([6]), 0.1, 0.0)
    assert np.allclose(o[0], np.repeat(c[sel[0]].mean(axis=0)[None], 4, 0), rtol=1e-13, atol=1e-16)
    assert np.allclose(lse[0], math.log(6), rtol=1e-14)


@pytest.mark.parametrize("rope_dim", [64, 0])
def test_mla_full_selection_equals_library_attention(rope_dim):
    """top_k >= context: sparse MLA over all keys equals torch's float64 scaled-dot-product
    attention with keys [c | kr] and values c (an independent library routine)."""
    n, H = 77, 8
    s, pool, q = _random_latent_case(n, H, rope_dim, 5)
    scale = 1.0 / math.sqrt(512 + rope_dim)
    idx = np.arange(96)
    idx[n:] = -1
    o, lse = O.sparse_mla(s, pool, "fp8", q, rope_dim, idx[None], np.array([n]), scale, 0.0)
    od, lsed = O.dense_mla(s, pool, "fp8", q, rope_dim, scale, 0.0)
    c, kr = O.latent_rows_fp8(pool, O.slots(s, 0, np.arange(n)), rope_dim)
    K = torch.from_numpy(np.concatenate([c, kr], axis=1))[None, None].expand(1, H, n, -1)
    V = torch.from_numpy(c)[None, None].expand(1, H, n, -1)
    Q = torch.from_numpy(O.decode_bf16(q[0]))[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0].numpy()
    assert np.allclose(o[0], ref, rtol=1e-10, atol=1e-13)
    assert np.allclose(od[0], ref, rtol=1e-10, atol=1e-13)
    logits = scale * (Q[0, :, 0] @ K[0, 0].T).numpy()
    assert np.allclose(lse[0], torch.logsumexp(torch.from_numpy(logits), dim=1).numpy(), rtol=1e-13)
    assert np.allclose(lsed[0], lse[0], rtol=1e-13)


@pytest.mark.parametrize("rope_dim", [64, 0])
def test_dense_mla_f32_and_plain_e4m3_formats_equal_library_attention(rope_dim):
    """dense_mla's fp32 and plain-E4M3 branches (queries times per-head scales, rows times
    the per-tensor scale) against torch's float64 scaled-dot-product attention on the
    decoded values, and against sparse_mla with every visible key selected."""
    g = np.random.default_rng(51)
    n, H = 45, 6
    seqs = O.Seqs(np.array([n]), np.array([0, 2]), np.array([30, n - 1]),
                  np.arange(1)[None, :], n)
    scale = 1.0 / math.sqrt(512 + rope_dim)
    rows32 = g.normal(size=(1, n, 576)).astype(np.float32)
    q32 = g.normal(size=(2, H, 512 + rope_dim)).astype(np.float32)
    codes = g.integers(0, 256, (1, n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x05
    qc = g.integers(0, 256, (2, H, 512 + rope_dim)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x3A
    qs = g.uniform(0.01, 0.02, size=(2, H))
    kv_scale = 0.0123
    cases = [("f32", rows32, q32, {},
              rows32[0].astype(np.float64), q32.astype(np.float64)),
             ("e4m3", codes, qc, {"q_scale": qs, "kv_scale": kv_scale},
              O.E4M3_TABLE[codes[0]] * kv_scale, O.E4M3_TABLE[qc] * qs[..., None])]
    for fmt, pool, q, kw, rows_v, q_v in cases:
        od, ld_ = O.dense_mla(seqs, pool, fmt, q, rope_dim, scale, 0.0, **kw)
        idx, ln = O.window_positions(seqs.q_pos, 64)
        os_, ls_ = O.sparse_mla(seqs, pool, fmt, q, rope_dim, idx, ln, scale, 0.0, **kw)
        assert np.allclose(od, os_, rtol=1e-12, atol=1e-14) and np.allclose(ld_, ls_, rtol=1e-13)
        for r in range(2):
            m = int(seqs.q_pos[r]) + 1
            K = torch.from_numpy(np.concatenate([rows_v[:m, :512], rows_v[:m, 512:512 + rope_dim]],
                                                axis=1))[None, None].expand(1, H, m, -1)
            V = torch.from_numpy(np.ascontiguousarray(rows_v[:m, :512]))[None, None].expand(1, H, m, -1)
            Q = torch.from_numpy(np.ascontiguousarray(q_v[r]))[None, :, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)[0, :, 0]
            assert np.allclose(od[r], ref.numpy(), rtol=1e-10, atol=1e-12), fmt
            lref = torch.logsumexp(scale * (Q[0, :, 0] @ K[0, 0].T), dim=1).numpy()
            assert np.allclose(ld_[r], lref, rtol=1e-12), fmt
    with pytest.raises(ValueError):
        O.dense_mla(seqs, codes, "e4m3", qc, rope_dim, scale, 0.0)          # no q_scale
    with pytest.raises(ValueError):
        O.dense_mla(seqs, rows32, "fp16", q32, rope_dim, scale, 0.0)        # unknown format
    with pytest.raises(ValueError):
        O.sparse_mla(seqs, rows32, "fp16", q32, rope_dim, np.zeros((2, 1), np.int64),
                     np.ones(2, np.int64), scale, 0.0)


def test_mla_ssmax_and_order_invariance_and_nope_rope_bytes():
    n, H = 50, 4
    s, pool, q = _random_latent_case(n, H, 64, 9)
    sel = np.array([[1, 4, 9, 16, 25, 36, 49, -1]])
    ln = np.array([7])
    base_o, base_l = O.sparse_mla(s, pool, "fp8", q, 64, sel, ln, 0.05, 0.0)
    unit = 1.0 / math.log(n)                      # s * ln(p + 1) == 1 at p = n - 1
    o, l = O.sparse_mla(s, pool, "fp8", q, 64, sel, ln, 0.05, unit)
    assert np.allclose(o, base_o, rtol=1e-13) and np.allclose(l, base_l, rtol=1e-13)
    o2, l2 = O.sparse_mla(s, pool, "fp8", q, 64, sel, ln, 0.05, 2 * unit)   # = doubled scale
    o3, l3 = O.sparse_mla(s, pool, "fp8", q, 64, sel, ln, 0.10, 0.0)
    assert np.allclose(o2, o3, rtol=1e-13) and np.allclose(l2, l3, rtol=1e-13)
    shuffled = np.array([[49, 9, 1, 36, 4, 25, 16, -1]])
    o4, l4 = O.sparse_mla(s, pool, "fp8", q, 64, shuffled, ln, 0.05, 0.0)
    assert np.allclose(o4, base_o, rtol=1e-13) and np.allclose(l4, base_l, rtol=1e-13)
    # NoPE: RoPE bytes are never read, even when they hold NaN
    q0 = q[:, :, :512].copy()
    a = O.sparse_mla(s, pool, "fp8", q0, 0, sel, ln, 0.05, 0.0)
    pool_nan = pool.copy()
    pool_nan.reshape(-1, 656)[:, 528:] = 0xFF
    b = O.sparse_mla(s, pool_nan, "fp8", q0, 0, sel, ln, 0.05, 0.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_mla_scale_groups_follow_latent_index():
    """Scale g multiplies codes 128*g .. 128*g + 127: code 1.0 at dims 0,128,256,384 with
    scales (1,2,4,8) dequantises to (1,2,4,8)."""
    s, nb = _one_request(1, bs=1)
    pool = P.latent_pool(nb, 1)
    P.put_latent_row(pool, 0, {0: 0x38, 128: 0x38, 256: 0x38, 384: 0x38, 127: 0x38},
                     [1.0, 2.0, 4.0, 8.0])
    c, _ = O.latent_rows_fp8(pool, np.array([0]), 64)
    assert c[0, [0, 127, 128, 256, 384]].tolist() == [1.0, 1.0, 2.0, 4.0, 8.0]
    assert np.count_nonzero(c[0]) == 5


def test_layer_modes_consumer_and_shared_indexer():
    rng = np.random.default_rng(2)
    n, H, Hi, bs = 60, 4, 3, 8
    s, pool0, q = _random_latent_case(n, H, 64, 21, bs=bs)
    _, pool1, _ = _random_latent_case(n, H, 64, 22, bs=bs)
    nb = pool0.shape[0]
    ipool = rng.integers(0, 256, size=(nb, bs, 132), dtype=np.uint8)
    ipool[:, :, :128][(ipool[:, :, :128] & 0x7F) == 0x7F] = 0
    ipool.reshape(-1, 132)[:, 128:] = np.frombuffer(np.ones(nb * bs, "<f4").tobytes(),
                                                    np.uint8).reshape(-1, 4)
    qi = rng.integers(0, 0x70, size=(1, Hi, 128), dtype=np.uint8)
    w = rng.uniform(size=(1, Hi))
    store = {}
    L0 = O.Layer(0, top_k=16)
    o0, l0, i0, n0 = O.layer_step(L0, s, "fp8", {0: pool0, 1: pool1}, {0: ipool, 2: ipool},
                                  qi, None, w, q, store, ld=64)
    assert 0 in store and n0[0] == 16
    L1 = O.Layer(1, topk_source_layer=0, top_k=16)           # own latent, L0's top-k
    o1, l1, i1, _ = O.layer_step(L1, s, "fp8", {0: pool0, 1: pool1}, {}, None, None, None,
                                 q, store, ld=64)
    assert np.array_equal(i1, i0) and 1 not in store
    ref1 = O.sparse_mla(s, pool1, "fp8", q, 64, i0, n0, L1.softmax_scale, 0.0)
    assert np.array_equal(o1, ref1[0]) and np.array_equal(l1, ref1[1])
    L2 = O.Layer(2, kv_sharing_target_layer=0, top_k=16)     # own indexer, L0's latent
    o2, l2, i2, _ = O.layer_step(L2, s, "fp8", {0: pool0, 1: pool1}, {2: ipool}, qi, None, w,
                                 q, store, ld=64)
    assert np.array_equal(o2, o0) and np.array_equal(i2, i0)   # same indexer inputs here


def test_consumer_layer_runs_its_own_indexer_on_the_owner_cache():
    """A KV-sharing consumer keeps its own indexer [blog, 跨层 KV 共享: only the latent cache
    is shared]: with indexer inputs unlike the owner's, its top-k is the top-k of its own
    scores (recomputed here from the definition, not taken from the owner), its attention
    reads the owner's latent rows, and a NaN-filled latent pool under its own layer number
    is never read."""
    n, H, Hi, bs, k = 96, 4, 2, 8, 12
    s, pool0, q = _random_latent_case(n, H, 64, 41, bs=bs)
    nb = pool0.shape[0]
    g = np.random.default_rng(42)

    def ipool_of(seed):
        r = np.random.default_rng(seed)
        ip = r.integers(0, 256, size=(nb, bs, 132), dtype=np.uint8)
        ip[:, :, :128][(ip[:, :, :128] & 0x7F) == 0x7F] = 0
        ip.reshape(-1, 132)[:, 128:] = np.frombuffer(
            r.uniform(0.5, 2.0, nb * bs).astype("<f4").tobytes(), np.uint8).reshape(-1, 4)
        return ip

    ip0, ip2 = ipool_of(43), ipool_of(44)
    qi0 = g.integers(0, 0x70, size=(1, Hi, 128), dtype=np.uint8)
    qi2 = g.integers(0, 0x70, size=(1, Hi, 128), dtype=np.uint8)
    w0, w2 = g.uniform(size=(1, Hi)), g.uniform(size=(1, Hi))
    nan_pool = np.full_like(pool0, 0x7F)                       # every code NaN
    lat = {0: pool0, 2: nan_pool}
    store = {}
    o0, l0, i0, n0 = O.layer_step(O.Layer(0, top_k=k), s, "fp8", lat, {0: ip0}, qi0, None, w0,
                                  q, store, ld=n)
    L2 = O.Layer(2, kv_sharing_target_layer=0, top_k=k)
    o2, l2, i2, n2 = O.layer_step(L2, s, "fp8", lat, {2: ip2}, qi2, None, w2, q, store, ld=n)
    # the consumer's own selection, from its own scores by brute-force sorting
    p = int(s.q_pos[0])
    sc = np.zeros(p + 1)
    for t in range(p + 1):
        kv, ks = O.index_rows_fp8(ip2, O.slots(s, 0, np.array([t])))
        dots = O.decode_e4m3(qi2[0]) @ kv[0]
        sc[t] = ks[0] * float(np.sum(w2[0] * np.maximum(dots, 0.0)))
    want = sorted(sorted(range(p + 1), key=lambda t: (-sc[t], t))[:k])
    assert list(i2[0][:k]) == want and n2[0] == k
    assert not np.array_equal(i2, i0), "inputs chosen so that the two selections differ"
    assert 2 in store and np.array_equal(store[2][0], i2)
    ref = O.sparse_mla(s, pool0, "fp8", q, 64, i2, n2, L2.softmax_scale, 0.0)
    assert np.array_equal(o2, ref[0]) and np.array_equal(l2, ref[1])
    assert np.all(np.isfinite(o2)) and not np.allclose(o2, o0)


# ---------------------------------------------------------------- KV-cache writes (quantiser)
def _e4m3_grid():
    vals = np.array(sorted({float(v) for v in O.E4M3_TABLE if np.isfinite(v) and v >= 0}))
    return vals


def test_e4m3_encoder_matches_torch_round_to_nearest_even():
    """Every finite E4M3 value, every midpoint between neighbours (ties), a quarter either
    side of each midpoint, and random binary32 values in range: the encoder's codes equal
    torch's float8_e4m3fn cast (round to nearest, ties to even) bit for bit."""
    pos = _e4m3_grid()
    mids = (pos[:-1] + pos[1:]) / 2
    quarter = (pos[1:] - pos[:-1]) / 4
    g = np.random.default_rng(3)
    rnd = g.uniform(-448, 448, 20000)
    small = g.uniform(-2.0 ** -5, 2.0 ** -5, 5000)
    x = np.concatenate([pos, -pos, mids, -mids, mids - quarter, mids + quarter,
                        -(mids + quarter), rnd, small]).astype(np.float32)
    got = O.encode_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    # decoding the code returns an exactly representable value unchanged
    assert np.array_equal(O.decode_e4m3(O.encode_e4m3(pos.astype(np.float32))), pos)


def test_e4m3_encoder_ties_go_to_even_codes():
    assert list(O.encode_e4m3(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 272.0],
                                       dtype=np.float32))) == [0x38, 0x3A, 0x00, 0x02, 0x78]
    assert O.encode_e4m3(np.array([-0.0], dtype=np.float32))[0] == 0x80


def test_index_row_quantiser_layout_scale_and_error_bound():
    g = np.random.default_rng(5)
    k = (g.standard_normal((64, 128)) * np.exp(g.uniform(-6, 6, (64, 1)))).astype(np.float32)
    k[3] = 0.0                                            # all-zero key
    rows = O.quantise_index_rows(k)
    assert rows.shape == (64, 132)
    codes, scale = rows[:, :128], rows[:, 128:].copy().view("<f4")[:, 0]
    amax = np.abs(k).max(axis=1).astype(np.float32)
    assert np.array_equal(scale, (amax / np.float32(448.0)).astype(np.float32))
    assert np.all(codes[3] == 0) and scale[3] == 0
    # the largest element of every non-zero key lands on +-448
    live = amax > 0
    top = np.abs(k).argmax(axis=1)
    assert np.all(np.isin(codes[live, top[live]], [0x7E, 0xFE]))
    # dequantised error: half an E4M3 step (2^-4 relative, 2^-10 absolute below 2^-6)
    deq = O.decode_e4m3(codes) * scale[:, None]
    bound = np.maximum(np.abs(k) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(deq - k) <= bound)
    # the indexer reader decodes what the writer packed
    pool = rows.reshape(1, 64, 132)
    kk, ks = O.index_rows_fp8(pool, np.arange(64))
    assert np.allclose(kk * ks[:, None], deq, rtol=0, atol=0)


def test_latent_row_quantiser_groups_rope_and_reader_round_trip():
    g = np.random.default_rng(6)
    c = (g.standard_normal((16, 512)) * np.repeat(np.exp(g.uniform(-4, 4, (16, 4))), 128, axis=1)
         ).astype(np.float32)
    c[5, 128:256] = 0.0                                   # one all-zero scale group
    rope = P.bf16_bits(torch.randn(16, 64, generator=torch.Generator().manual_seed(2)))
    rows = O.quantise_latent_rows(c, rope)
    assert rows.shape == (16, 656)
    scales = rows[:, 512:528].copy().view("<f4")
    for gi in range(4):
        amax = np.abs(c[:, 128 * gi:128 * (gi + 1)]).max(axis=1).astype(np.float32)
        assert np.array_equal(scales[:, gi], (amax / np.float32(448.0)).astype(np.float32))
    assert scales[5, 1] == 0 and np.all(rows[5, 128:256] == 0)
    assert np.array_equal(rows[:, 528:].copy().view("<u2"), rope.astype(np.uint16))
    cc, kr = O.latent_rows_fp8(rows.reshape(1, 16, 656), np.arange(16), 64)
    bound = np.maximum(np.abs(c) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scales, 128, axis=1))
    assert np.all(np.abs(cc - c) <= bound * (1 + 1e-6))
    assert np.array_equal(kr, O.decode_bf16(rope))
    # without RoPE input the RoPE bytes stay untouched (zero here)
    assert np.all(O.quantise_latent_rows(c[:2], None)[:, 528:] == 0)


# ---------------------------------------------------------------- split-context merge
@pytest.mark.parametrize("seed", range(12))
def test_topk_merge_of_chunk_topks_equals_row_topk(seed):
    """Top-k of the union of per-chunk top-k lists is the row's top-k (every key of the
    row's top-k is in its chunk's top-k), with duplicates, -0, -inf and NaN in the row."""
    g = np.random.default_rng(seed)
    n = int(g.integers(50, 400))
    k = int(g.integers(1, 40))
    x = np.round(g.standard_normal(n) * 3) / 3
    x[g.integers(0, n, 5)] = -0.0
    x[g.integers(0, n, 3)] = -np.inf
    x[g.integers(0, n, 2)] = np.nan
    S = int(g.integers(1, 9))
    bounds = np.linspace(0, n, S + 1).astype(int)
    cs, cp, cl = np.zeros((S, k)), np.full((S, k), -1), np.zeros(S, dtype=int)
    for s_ in range(S):
        lo, hi = bounds[s_], bounds[s_ + 1]
        if hi > lo:
            idx, ln = O.topk_row(x[lo:hi], hi - lo - 1, k)
            cs[s_, :ln], cp[s_, :ln], cl[s_] = x[lo + idx[:ln]], lo + idx[:ln], ln
    got, gl = O.topk_merge(cs, cp, cl, k)
    want, wl = O.topk_row(x, n - 1, k)
    assert gl == wl and np.array_equal(got, want)


def test_topk_merge_brute_force_order():
    cs = np.array([[3.0, 1.0, 0.0], [3.0, 2.0, -0.0]])
    cp = np.array([[7, 2, 5], [4, 9, 1]])
    got, n = O.topk_merge(cs, cp, np.array([3, 3]), 4)
    # 3.0@4 and 3.0@7 (tie: lower position first), 2.0@9, 1.0@2 -> ascending positions
    assert n == 4 and list(got) == [2, 4, 7, 9]
    got, n = O.topk_merge(cs, cp, np.array([1, 0]), 4)
    assert n == 1 and list(got) == [7, -1, -1, -1]


def test_lse_combine_of_split_attention_equals_full_attention():
    """Attention over disjoint key subsets, merged by LSE, equals attention over all keys
    (torch float64 softmax as the independent reference)."""
    g = torch.Generator().manual_seed(4)
    H, D, n, S = 6, 16, 50, 4
    q = torch.randn(H, D, generator=g, dtype=torch.float64)
    kv = torch.randn(n, D, generator=g, dtype=torch.float64)
    logits = q @ kv.T * 0.7
    full = torch.softmax(logits, dim=1) @ kv
    full_lse = torch.logsumexp(logits, dim=1)
    parts = torch.randperm(n, generator=g).chunk(S - 1)
    o_parts, lse_parts = [], []
    for p in parts:
        l = logits[:, p]
        o_parts.append((torch.softmax(l, dim=1) @ kv[p]).numpy())
        lse_parts.append(torch.logsumexp(l, dim=1).numpy())
    o_parts.append(np.zeros((H, D)))                 # an empty shard
    lse_parts.append(np.full(H, -np.inf))
    o, lse = O.lse_combine(np.stack(o_parts), np.stack(lse_parts))
    assert np.allclose(o, full.numpy(), atol=1e-12) and np.allclose(lse, full_lse.numpy())
    o, lse = O.lse_combine(np.zeros((2, H, D)), np.full((2, H), -np.inf))
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- bf16 rows, sliding window
def test_bf16_rows_and_window_selection_reduce_to_dense_attention():
    """bf16 latent rows read back as their values; a window covering the whole context is
    dense attention; the window positions are the trailing ones, clipped at 0."""
    g = torch.Generator().manual_seed(9)
    rows = torch.randn(1, 16, 576, generator=g).to(torch.bfloat16)
    bits = P.bf16_bits(rows.float())
    seqs = O.Seqs(np.array([16]), np.array([0, 2]), np.array([9, 15]), np.arange(1)[None, :], 16)
    c, kr = O.latent_rows_bf16(bits, np.arange(16), 64)
    assert np.array_equal(c, rows.float().numpy()[0, :, :512].astype(np.float64))
    assert np.array_equal(kr, rows.float().numpy()[0, :, 512:].astype(np.float64))
    idx, ln = O.window_positions(np.array([9, 15, 2]), 4)
    assert list(idx[0]) == [6, 7, 8, 9] and list(idx[2]) == [0, 1, 2, -1] and list(ln) == [4, 4, 3]
    q = P.bf16_bits(torch.randn(2, 4, 576, generator=g))
    widx, wln = O.window_positions(seqs.q_pos, 64)
    o, lse = O.sparse_mla(seqs, bits, "bf16", q, 64, widx, wln, 0.05, 0.0)
    od, lsed = O.dense_mla(seqs, bits, "bf16", q, 64, 0.05, 0.0)
    assert np.allclose(o, od, atol=1e-12) and np.allclose(lse, lsed)


def test_plain_e4m3_rows_equal_fp8_ds_mla_rows_with_uniform_power_of_two_scales():
    """A plain E4M3 576-B row with per-tensor scale 2^-5 and an FP8 query with scales 2^-3
    are the same values as an fp8_ds_mla row whose four group scales are 2^-5 and whose
    bf16 RoPE holds the decoded RoPE codes times 2^-5, with a bf16 query of the decoded
    codes times 2^-3 (all exact): attention over both is identical."""
    g = np.random.default_rng(10)
    n, H = 40, 4
    codes = g.integers(0, 256, (n, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00                    # no NaN codes
    ks = 2.0 ** -5
    plain = codes.reshape(1, n, 576)
    ds = np.zeros((1, n, 656), dtype=np.uint8)
    ds[0, :, :512] = codes[:, :512]
    ds[0, :, 512:528] = np.frombuffer(np.full(4 * n, ks, dtype="<f4").tobytes(),
                                      dtype=np.uint8).reshape(n, 16)
    rope_vals = O.decode_e4m3(codes[:, 512:]) * ks
    ds[0, :, 528:] = P.bf16_bits(rope_vals.astype(np.float32)).view(np.uint8).reshape(n, 128)
    qc = g.integers(0, 256, (2, H, 576)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x38
    qs = np.full((2, H), 2.0 ** -3)
    qbf = P.bf16_bits((O.decode_e4m3(qc) * 2.0 ** -3).astype(np.float32))
    seqs = O.Seqs(np.array([n]), np.array([0, 2]), np.array([30, 39]), np.arange(1)[None, :], n)
    idx, ln = O.window_positions(seqs.q_pos, 64)
    for rope in (64, 0):
        a = O.sparse_mla(seqs, plain, "e4m3", qc[..., :512 + rope], rope, idx, ln, 0.05, 0.3,
                         q_scale=qs, kv_scale=ks)
        b = O.sparse_mla(seqs, ds, "fp8", qbf[..., :512 + rope], rope, idx, ln, 0.05, 0.3)
        assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], atol=1e-12)


def test_bf16_encoder_matches_torch_round_to_nearest_even():
    """Random binary32 values over many binades, exact bf16 values, and every tie pattern
    (low half 0x8000 with even and odd kept halves): the bits equal torch's float32 ->
    bfloat16 cast."""
    g = np.random.default_rng(11)
    x = (g.standard_normal(20000) * np.exp(g.uniform(-30, 30, 20000))).astype(np.float32)
    base = g.integers(0, 0x7F7F, 4000, dtype=np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001]).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, -0.0, 1.0, 3.0e38])]).astype(np.float32)
    got = O.encode_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_second_layout_writers_round_trip_through_their_readers():
    """bf16 rows read back as the bf16-rounded latents and the RoPE bits as given; plain-E4M3
    rows equal torch's float8_e4m3fn cast of clamp(x / kv_scale) in binary32 and read back
    within half an E4M3 step (saturated beyond 448 * kv_scale)."""
    g = np.random.default_rng(12)
    c = (g.standard_normal((8, 512)) * 3).astype(np.float32)
    c[0, :4] = [1000.0, -1000.0, 0.0, -0.0]                  # saturating and signed zeros
    rope = (g.standard_normal((8, 64))).astype(np.float32)
    rope_bits = O.encode_bf16(rope)
    rows16 = O.pack_latent_rows_bf16(c, rope_bits)
    cc, kr = O.latent_rows_bf16(rows16.reshape(1, 8, 576), np.arange(8), 64)
    assert np.array_equal(cc, torch.from_numpy(c).to(torch.bfloat16).double().numpy())
    assert np.array_equal(kr, O.decode_bf16(rope_bits))
    kv_scale = 4.5 / 448
    rows8 = O.quantise_latent_rows_e4m3(c, O.decode_bf16(rope_bits), kv_scale)
    s32 = np.float32(kv_scale)
    ref_c = torch.from_numpy(np.clip(c / s32, -448, 448).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rows8[:, :512], ref_c)
    cc8, kr8 = O.latent_rows_e4m3(rows8.reshape(1, 8, 576), np.arange(8), 64, kv_scale)
    inside = np.abs(c) <= 448 * kv_scale
    bound = np.maximum(np.abs(c) * 2.0 ** -4, 2.0 ** -10 * kv_scale) * (1 + 1e-6)
    assert np.all(np.abs(cc8 - c)[inside] <= bound[inside])
    assert np.all(np.abs(cc8[~inside]) == 448 * kv_scale)
    assert np.all(np.abs(kr8 - O.decode_bf16(rope_bits)) <= np.maximum(
        np.abs(O.decode_bf16(rope_bits)) * 2.0 ** -4, 2.0 ** -10 * kv_scale) * (1 + 1e-6))


def test_fp32_format_readers_agree_with_fp8_formats_on_exact_values():
    """The fp32 cache format (the tiny fp32 decode workload) has its own row readers; holding
    the exact values of fp8 rows (power-of-two scales, so code x scale is exact in binary32)
    it must give the fp8 formats' indexer scores and attention.  Pins the fp32 readers and
    the fp32 query path to the separately pinned fp8 ones."""
    rng = np.random.default_rng(31)
    H, n, bs = 5, 37, 8
    s, nb = _one_request(n, bs=bs)
    # indexer: e4m3 keys with a power-of-two scale per key, e4m3 queries with power-of-two
    # per-head scales
    ipool = P.index_pool(nb, bs)
    flat = ipool.reshape(-1, 132)
    codes = rng.integers(0, 256, size=(nb * bs, 128), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x22
    flat[:, :128] = codes
    ks = np.exp2(rng.integers(-6, 3, size=nb * bs)).astype(np.float32)
    flat[:, 128:] = np.frombuffer(ks.astype("<f4").tobytes(), np.uint8).reshape(-1, 4)
    qc = rng.integers(0, 256, size=(1, H, 128), dtype=np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x41
    qs = np.exp2(rng.integers(-4, 4, size=(1, H))).astype(np.float32)
    w = rng.uniform(-1, 1, size=(1, H)).astype(np.float32)
    ref = O.indexer_scores(s, ipool, "fp8", qc, qs, w, 0.25, n)
    kf = (O.decode_e4m3(codes) * ks[:, None]).astype(np.float32)            # exact
    ipool32 = kf.reshape(nb, bs, 128)
    q32 = (O.decode_e4m3(qc) * qs[..., None]).astype(np.float32)            # exact
    got = O.indexer_scores(s, ipool32, "f32", q32, None, w, 0.25, n)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    # attention: fp8_ds_mla rows with power-of-two group scales, bf16 RoPE, bf16 queries
    s2, pool, q = _random_latent_case(n, H, 64, 32)
    lat = pool.reshape(-1, 656)
    sc = np.exp2(rng.integers(-9, -4, size=(lat.shape[0], 4))).astype("<f4")
    lat[:, 512:528] = np.frombuffer(sc.tobytes(), np.uint8).reshape(-1, 16)
    sel = np.array([[0, 3, 8, 9, 20, 36, -1, -1]])
    ln = np.array([6])
    o8, l8 = O.sparse_mla(s2, pool, "fp8", q, 64, sel, ln, 0.05, 0.3)
    c, kr = O.latent_rows_fp8(pool, np.arange(lat.shape[0]), 64)
    pool32 = np.concatenate([c, kr], axis=1).astype(np.float32).reshape(pool.shape[0], pool.shape[1], 576)
    assert np.array_equal(pool32.reshape(-1, 576).astype(np.float64), np.concatenate([c, kr], 1))
    q32m = O.decode_bf16(q).astype(np.float32)
    o32, l32 = O.sparse_mla(s2, pool32, "f32", q32m, 64, sel, ln, 0.05, 0.3)
    assert np.allclose(o32, o8, rtol=1e-12, atol=1e-15)
    assert np.allclose(l32, l8, rtol=1e-12, atol=0)
