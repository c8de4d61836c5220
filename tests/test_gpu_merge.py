"""Split-context merge entries against the oracle (MI355X only), and their composition with
the path: per-shard attention over a row's selected keys merged by LSE equals attention over
all of them."""

import math

import numpy as np
import pytest
import torch

import oracle as O
from tests.compare import batch_np, check_close, t_np

pytestmark = pytest.mark.gpu

M = pytest.importorskip("sparse_attention_decode_dsa_amd.ml4dsa")
from sparse_attention_decode_dsa_amd import synth  # noqa: E402

DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _candidates(rows, S, ld, seed, with_nan):
    g = np.random.default_rng(seed)
    sc = np.round(g.standard_normal((rows, S, ld)) * 4).astype(np.float32) / 4   # many ties
    pos = np.full((rows, S, ld), -1, dtype=np.int32)
    ln = g.integers(0, ld + 1, (rows, S)).astype(np.int32)
    ln[0, 0] = ld
    for r in range(rows):
        p = g.permutation(1 << 20)[:S * ld].reshape(S, ld)      # distinct positions per row
        pos[r] = p
    sc[0, 0, 3] = -0.0
    sc[0, 0, 4] = 0.0
    sc[1 % rows, 0, 0] = -np.inf
    if with_nan:
        sc[0, 0, 5] = np.nan
    return sc, pos, ln


@pytest.mark.parametrize("rows,S,ld,k", [(4, 8, 2048, 2048), (3, 1, 1000, 777), (2, 16, 1024, 64),
                                         (3, 5, 300, 2048)])
def test_topk_merge_matches_oracle(rows, S, ld, k):
    print(f"[gpu] topk merge rows={rows} S={S} ld={ld} k={k}", flush=True)
    sc, pos, ln = _candidates(rows, S, ld, rows * 100 + S, with_nan=S > 1)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    olen = torch.zeros(rows, dtype=torch.int32, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    M.ml4_topk_merge(rows, S, torch.from_numpy(sc).to(DEV), torch.from_numpy(pos).to(DEV),
                     torch.from_numpy(ln).to(DEV), ld, k, idx, olen, fault)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == (M.ML4_FAULT_NAN_SCORE if S > 1 else 0)
    gi, gl = t_np(idx), t_np(olen)
    for r in range(rows):
        want, n = O.topk_merge(sc[r], pos[r], ln[r], k)
        assert gl[r] == n
        assert np.array_equal(gi[r], want)


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_lse_combine_matches_oracle(out_dtype):
    print(f"[gpu] lse combine {out_dtype}", flush=True)
    g = np.random.default_rng(8)
    rows, S, H, D = 3, 6, 16, 512
    o = g.standard_normal((rows, S, H, D)).astype(np.float32)
    lse = (g.standard_normal((rows, S, H)) * 5).astype(np.float32)
    lse[0, 2] = -np.inf                          # an empty shard
    lse[1, :, 3] = -np.inf                       # a head with no key anywhere
    dt = M.ML4_BF16 if out_dtype == "bf16" else M.ML4_F32
    out = torch.zeros(rows, H, D, dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                      device=DEV)
    olse = torch.zeros(rows, H, dtype=torch.float32, device=DEV)
    M.ml4_lse_combine(rows, H, S, D, torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV),
                      out, dt, olse)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for r in range(rows):
        wo, wl = O.lse_combine(o[r], lse[r])
        check_close(got[r], wo, f"row {r}")
        assert np.allclose(olse.cpu().numpy()[r], wl, rtol=1e-6, atol=1e-5, equal_nan=False) or \
            np.array_equal(np.isinf(olse.cpu().numpy()[r]), np.isinf(wl))


def test_split_context_attention_merges_to_the_whole():
    """A row's selected keys split by position across 4 context shards: sparse MLA per
    shard (with lse), merged by ml4_lse_combine, matches the oracle's attention over all
    selected keys; the shards' top-k lists merged by ml4_topk_merge equal the row's top-k."""
    print("[gpu] split-context composition", flush=True)
    case = synth.make_case("dcp", 71, seq_lens=[6000], q_per_seq=[2], block_size=64, fmt="fp8",
                           idx_heads=64, mla_heads=128, layers=[synth.layer_desc(0, ssmax_s=0.3)])
    c = synth.case_to(case, DEV)
    b = c.batch
    seqs = M.make_seqs(b)
    li = c.inputs[0]
    d = case.layers[0]
    K, H, T = d["top_k"], case.mla_heads, b.total_q
    n = int(b.seq_lens.max().item())
    ld = (n + 3) // 4 * 4
    scores = torch.empty(T, ld, dtype=torch.float32, device=DEV)
    fault = torch.zeros(1, dtype=torch.int32, device=DEV)
    icache = M.make_cache(li.idx_pool, M.ML4_IDX_FP8_132)
    M.ml4_indexer_score(seqs, icache, li.q_idx, M.ML4_FP8_E4M3, li.q_idx_scale, li.w_idx, 64,
                        d["idx_ssmax_s"], scores, ld, fault)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    ln = torch.empty(T, dtype=torch.int32, device=DEV)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_TOPK, seqs, 0, K)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=DEV)
    M.ml4_topk_select(seqs, scores, ld, K, idx, ln, ws, wsn, fault)
    torch.cuda.synchronize()
    # per-shard candidate lists: the shard's positions of the row's scores, top-K of each
    S = 4
    bounds = np.linspace(0, n, S + 1).astype(int)
    sc_np = scores.cpu().numpy()
    qpos = b.q_pos.cpu().numpy()
    cs = np.zeros((T, S, K), np.float32)
    cp = np.full((T, S, K), -1, np.int32)
    cl = np.zeros((T, S), np.int32)
    for r in range(T):
        for s_ in range(S):
            lo, hi = bounds[s_], min(bounds[s_ + 1], qpos[r] + 1)
            if hi <= lo:
                continue
            seg = sc_np[r, lo:hi]
            order = np.lexsort((np.arange(hi - lo), -seg))[:K]
            cl[r, s_] = len(order)
            cs[r, s_, :len(order)] = seg[order]
            cp[r, s_, :len(order)] = lo + order
    midx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    mlen = torch.empty(T, dtype=torch.int32, device=DEV)
    M.ml4_topk_merge(T, S, torch.from_numpy(cs).to(DEV), torch.from_numpy(cp).to(DEV),
                     torch.from_numpy(cl).to(DEV), K, K, midx, mlen, fault)
    torch.cuda.synchronize()
    assert np.array_equal(t_np(midx), t_np(idx)) and np.array_equal(t_np(mlen), t_np(ln))
    # attention per shard over the row's selected keys that fall in the shard
    sel = t_np(idx)
    lcache = M.make_cache(li.lat_pool, M.ML4_LAT_FP8_656)
    o_parts = np.zeros((T, S, H, 512), np.float32)
    l_parts = np.zeros((T, S, H), np.float32)
    for s_ in range(S):
        part = np.full_like(sel, -1)
        plen = np.zeros(T, np.int32)
        for r in range(T):
            v = sel[r][(sel[r] >= bounds[s_]) & (sel[r] < bounds[s_ + 1])]
            part[r, :len(v)] = v
            plen[r] = len(v)
        o = torch.empty(T, H, 512, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(T, H, dtype=torch.float32, device=DEV)
        mws = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, seqs, H, K)
        mw = torch.empty(max(mws, 256), dtype=torch.uint8, device=DEV)
        M.ml4_sparse_mla_decode(seqs, lcache, li.q_mla, M.ML4_BF16, H, 64,
                                torch.from_numpy(part.astype(np.int32)).to(DEV),
                                torch.from_numpy(plen).to(DEV), K, d["softmax_scale"], d["ssmax_s"],
                                o, M.ML4_BF16, lse, mw, mws, fault)
        torch.cuda.synchronize()
        o_parts[:, s_] = o.float().cpu().numpy()
        l_parts[:, s_] = lse.cpu().numpy()
    out = torch.empty(T, H, 512, dtype=torch.float32, device=DEV)
    M.ml4_lse_combine(T, H, S, 512, torch.from_numpy(o_parts).to(DEV),
                      torch.from_numpy(l_parts).to(DEV), out, M.ML4_F32, None)
    torch.cuda.synchronize()
    assert M.ml4_fault_query(fault) == 0
    seqs_o = batch_np(case.batch)
    ref, _ = O.sparse_mla(seqs_o, t_np(case.inputs[0].lat_pool), "fp8",
                          t_np(case.inputs[0].q_mla), 64, sel, t_np(ln), d["softmax_scale"],
                          d["ssmax_s"])
    check_close(out.cpu().numpy(), ref, "split-context attention")
