"""The no-allocation fused entry (library-held scratch) against the fused entry with a
caller workspace, through the C ABI: two calls in a row on one GPU, the second with a
smaller batch, every output bit-identical (same kernels, same inputs)."""

import pytest
import torch

pytestmark = pytest.mark.gpu

M = pytest.importorskip("sparse_attention_decode_dsa_amd.ml4dsa")
from sparse_attention_decode_dsa_amd import synth  # noqa: E402
from sparse_attention_decode_dsa_amd.runner import CaseRunner  # noqa: E402

DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _outputs(run):
    return ([t.clone() for l in sorted(run.out) for t in (run.out[l], run.lse[l])] +
            [t.clone() for l in sorted(run.topk_idx)
             for t in (run.topk_idx[l], run.topk_len[l])])


def _poison(run):
    for l in run.out:
        run.out[l].fill_(float("nan"))
        run.lse[l].fill_(float("nan"))
    for l in run.topk_idx:
        run.topk_idx[l].fill_(-7)
        run.topk_len[l].fill_(-7)


def _bytes(t):
    return t.contiguous().view(torch.uint8)


def test_static_scratch_entry_matches_workspace_entry_on_two_calls():
    L = synth.layer_desc
    # first call: two rows past 131,072 positions (the long-row top-k keeps its per-chunk
    # candidate lists and their lengths in the scratch) and few rows (split-MLA partials
    # in the scratch), owner / shared-indexer / consumer layers
    big = synth.make_case(
        "na_big", 91, seq_lens=[140001, 150000], q_per_seq=[1, 1], block_size=64, fmt="fp8",
        idx_heads=64, mla_heads=128,
        layers=[L(0, ssmax_s=0.3), L(1, topk_source_layer=0), L(2, kv_sharing_target_layer=0)],
        device=DEV)
    # second call: a smaller batch (short rows: the one-work-group top-k; fewer splits)
    small = synth.make_case(
        "na_small", 92, seq_lens=[3000, 777, 5001], q_per_seq=[1, 1, 2], block_size=64,
        fmt="fp8", idx_heads=64, mla_heads=128, layers=[L(0), L(1, rope_dim=0)], device=DEV)
    for case in (big, small):
        print(f"[no-alloc] {case.name}: rows {case.batch.total_q}, context "
              f"{case.batch.max_seq_len}, layers {[d['layer'] for d in case.layers]}",
              flush=True)
        run = CaseRunner(case)
        need = M.ml4_workspace_bytes(M.ML4_ENTRY_LAYER, run.seqs, case.mla_heads,
                                     case.layers[0]["top_k"])
        assert 0 < need <= M.ML4_STATIC_SCRATCH_BYTES
        for d in case.layers:
            run.run_layer_fused(d["layer"])
        torch.cuda.synchronize()
        assert run.fault_bits() == 0
        ref = _outputs(run)
        _poison(run)
        for d in case.layers:
            run.run_layer_static(d["layer"])
        torch.cuda.synchronize()
        assert run.fault_bits() == 0
        got = _outputs(run)
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(_bytes(a), _bytes(b)), (case.name, i)
        del run


def test_static_scratch_entry_refuses_a_batch_above_its_scratch():
    L = synth.layer_desc
    case = synth.make_case("na_over", 93, seq_lens=[65536] * 2, q_per_seq=[132, 130],
                           block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                           layers=[L(0)], device=DEV)
    run = CaseRunner(case)
    assert M.ml4_workspace_bytes(M.ML4_ENTRY_LAYER, run.seqs, 128, 2048) > \
        M.ML4_STATIC_SCRATCH_BYTES
    with pytest.raises(M.ML4Error) as e:
        run.run_layer_static(0)
    assert e.value.code == M.ML4_E_UNSUPPORTED
    assert "ML4_STATIC_SCRATCH_BYTES" in e.value.message
