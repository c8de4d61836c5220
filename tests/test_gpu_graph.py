"""A whole decode step captured into a HIP graph (torch.cuda.CUDAGraph) and replayed (MI355X
only).  The fused layer entry only launches kernels on the caller's stream, so a step can be
captured once and replayed with new inputs in the same buffers: every replay -- with eager
work and new inputs between replays -- must give outputs, LSEs and top-k lists bit-identical
to an eager run of the same entries on the same inputs."""

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


def _say(msg):
    print(msg, flush=True)


def _outputs(run):
    res = {}
    for l in run.out:
        res[("out", l)] = run.out[l].clone()
        res[("lse", l)] = run.lse[l].clone()
    for l in run.topk_idx:
        res[("idx", l)] = run.topk_idx[l].clone()
        res[("len", l)] = run.topk_len[l].clone()
    return res


def _clobber(run):
    for l in run.out:
        run.out[l].fill_(float("nan"))
        run.lse[l].fill_(float("nan"))
    for l in run.topk_idx:
        run.topk_idx[l].fill_(-7)
        run.topk_len[l].fill_(-7)


def _same(a, b):
    if a.dtype in (torch.int32, torch.int64):
        return bool(torch.equal(a, b))
    return bool(torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)))


def _new_inputs(case):
    """Next step's queries in the same buffers: each layer's query rows rotated by one."""
    for li in case.inputs.values():
        for t in (li.q_idx, li.q_idx_scale, li.w_idx, li.q_mla):
            if t is not None:
                t.copy_(torch.roll(t, 1, dims=0))


CASES = {
    # owner / shared-indexer / KV-sharing consumer, few rows: split MLA + merge kernel
    "decode_3layer": dict(seq_lens=[5000, 3000, 700], q_per_seq=[1, 1, 1],
                          layers=[synth.layer_desc(0),
                                  synth.layer_desc(1, topk_source_layer=0),
                                  synth.layer_desc(2, kv_sharing_target_layer=0,
                                                   ssmax_s=0.3)]),
    # rows longer than 131,072 positions: the multi-work-group top-k (six launches)
    "decode_long_row": dict(seq_lens=[140000], q_per_seq=[1], layers=[synth.layer_desc(0)]),
    # verify rows sharing each key scan, RoPE + NoPE layers
    "verify_2x4": dict(seq_lens=[9000, 4100], q_per_seq=[4, 4],
                       layers=[synth.layer_desc(0, ssmax_s=0.3),
                               synth.layer_desc(1, rope_dim=0, ssmax_s=0.3)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_step_replays_bit_identical(name):
    spec = CASES[name]
    _say(f"[gpu] graph capture {name}")
    case = synth.make_case(name, 5, seq_lens=spec["seq_lens"], q_per_seq=spec["q_per_seq"],
                           block_size=64, fmt="fp8", idx_heads=64, mla_heads=128,
                           layers=spec["layers"], device=DEV)
    run = CaseRunner(case)

    run.run_step(fused=True)
    torch.cuda.synchronize()
    ref = _outputs(run)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.run_step(fused=True)            # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.run_step(fused=True)
    torch.cuda.synchronize()

    for rep in range(4):
        if rep >= 2:                         # a new step: new queries, eager reference
            _new_inputs(case)
            run.run_step(fused=True)
            torch.cuda.synchronize()
            ref = _outputs(run)
        _clobber(run)
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(run)
        for key, want in ref.items():
            assert _same(got[key], want), (name, rep, key)
        _say(f"  replay {rep}: bit-identical")
    assert run.fault_bits() == 0
    del graph
