"""Benchmark of the sparse-attention step on one MI355X.

Workload (default): speculative-verify decode at 64k context -- 64 requests x 4 query rows,
context 65,536, paged 64-token blocks with a seeded random block table, indexer 64 heads x
128 on the 132-byte FP8 cache, top-2048, MLA 128 heads on the 656-byte FP8 latent cache,
SSMax s = 0.3; one RoPE layer and one NoPE layer per step.  Inputs are seeded synthetic
data drawn on the GPU and resident in HBM before timing starts.

One step = for each layer: indexer scores -> exact top-k -> sparse MLA (the three entry
points the fused entry chains), timed with HIP events on the launch stream.  Before each
timed step a streaming read of an unrelated 1 GiB buffer (outside the step's events) evicts
the memory-side cache and the L2s with clean lines, so the decode workloads whose caches
would fit in the 256 MB memory-side cache still read them from HBM, and no step pays for
write-backs of data it did not write; value is query rows over the mean step time, with
p10/p50/p90 and the back-to-back ("hot") time beside it.
Each kernel is reported against its floors at datasheet peaks and against the rates a
plain streaming read and a library GEMM reach on the same GPU.
Prints one JSON line.  --gpus N > 1 is refused: the benchmark runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode query-tokens/s + achieved HBM GB/s, sparse MLA+DSA at 64k context"
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
KERNEL_SOURCES = {"indexer": "indexer.hip", "topk": "topk.hip", "mla": "sparse_mla.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload 1..5 (3 = verify at 64k)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU budget of the oracle baseline sample (0 = skip)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB read + 1 GiB write streaming "
                         "kernel (counter calibration)")
    ap.add_argument("--cache-write-tokens", type=int, default=65536,
                    help="also time the KV-cache write entries on this many bf16 tokens "
                         "(0 = skip); reported beside the step, not in it")
    ap.add_argument("--no-layouts", action="store_true",
                    help="skip the side measurements of the bf16-row layout and of "
                         "sliding-window attention")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the side measurement of the step captured into a HIP graph")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable streaming and GEMM rates")
    ap.add_argument("--fused", action="store_true",
                    help="time the fused entry instead (no per-kernel events)")
    return ap.parse_args()


def kernel_hash(name: str) -> str:
    p = os.path.join(ROOT, "sparse_attention_decode_dsa_amd", "csrc", KERNEL_SOURCES[name])
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def algorithmic_work(case):
    """Per layer: indexer bytes (keys read once per request + queries), MLA bytes (selected
    latent rows + q + o) and MLA FLOPs, from the workload's shape.  The fp32 scores the
    indexer writes and the selection reads back (4 B per visible position per row) are an
    implementation overhead of the split path, reported apart as score_bytes."""
    b = case.batch
    seq = b.seq_lens.cpu().tolist()
    T, Hi, H = b.total_q, case.idx_heads, case.mla_heads
    qpos = b.q_pos.cpu().tolist()
    out = {}
    for d in case.layers:
        k = d["top_k"]
        nsel = [min(k, p + 1) for p in qpos]
        idx_bytes = 0
        score_bytes = 0
        if d["topk_source_layer"] < 0:
            # cache rows read once per request, fp8 query + fp32 scale + weight per head
            idx_bytes = sum(n * 132 for n in seq) + T * Hi * (128 + 8)
            # one fp32 score per (row, visible position): written once, read by the top-k
            score_bytes = sum(p + 1 for p in qpos) * 4
        rope = d["rope_dim"]
        row = 656 if rope else 528
        mla_bytes = sum(nsel) * row + T * H * (512 + rope) * 2 + T * H * 512 * 2
        mla_flops = sum(nsel) * 2 * H * (1024 + rope)
        # each row scores its visible positions 0 .. p (causal)
        idx_flops = sum(p + 1 for p in qpos) * 2 * Hi * 128 if d["topk_source_layer"] < 0 else 0
        out[d["layer"]] = dict(idx_bytes=idx_bytes, idx_flops=idx_flops, mla_bytes=mla_bytes,
                               mla_flops=mla_flops, score_bytes=score_bytes)
    return out


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the current
    kernel source and on this workload (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except Exception:
        return None
    if t.get("source_sha256_16") != kernel_hash(kernel) or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(case, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the workload's query rows."""
    import numpy as np
    import torch

    import oracle as O
    from tests.compare import t_np

    b = case.batch
    bs = b.block_size
    q_start = b.q_start.cpu().numpy()
    rows_done = 0
    t0 = time.perf_counter()
    sample = []
    r = 0
    # whole requests, all their rows, all layers, until the budget is spent
    for req in range(b.batch):
        if time.perf_counter() - t0 > budget_s and rows_done:
            break
        nblk = (int(b.seq_lens[req].item()) + bs - 1) // bs
        blocks = b.block_table[req, :nblk].long()
        seqs = O.Seqs(np.array([int(b.seq_lens[req].item())]), np.array([0, int(q_start[req + 1] - q_start[req])]),
                      b.q_pos[q_start[req]:q_start[req + 1]].cpu().numpy().astype(np.int64),
                      np.arange(nblk)[None, :], bs)
        rows = slice(int(q_start[req]), int(q_start[req + 1]))
        lat, idxp = {}, {}
        for d in case.layers:
            li = case.inputs[d["layer"]]
            if li.lat_pool is not None:
                lat[d["layer"]] = t_np(li.lat_pool[blocks])
            if li.idx_pool is not None:
                idxp[d["layer"]] = t_np(li.idx_pool[blocks])
        store = {}
        t_req = time.perf_counter()
        for d in case.layers:
            li = case.inputs[d["layer"]]
            L = O.Layer(d["layer"], d["kv_sharing_target_layer"], d["topk_source_layer"],
                        d["rope_dim"], d["top_k"], d["softmax_scale"], d["ssmax_s"],
                        d["idx_ssmax_s"])
            O.layer_step(L, seqs, case.fmt, lat, idxp,
                         None if li.q_idx is None else t_np(li.q_idx[rows]),
                         None if li.q_idx_scale is None else t_np(li.q_idx_scale[rows]),
                         None if li.w_idx is None else t_np(li.w_idx[rows]),
                         t_np(li.q_mla[rows]), store, ld=int(b.max_seq_len))
        sample.append(time.perf_counter() - t_req)
        rows_done += seqs.total_q
    elapsed = sum(sample)
    cores = None
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count()
    cpu_model = None
    sockets, phys = set(), set()
    try:
        with open("/proc/cpuinfo") as f:
            pid = None
            for line in f:
                if line.startswith("model name") and cpu_model is None:
                    cpu_model = line.split(":", 1)[1].strip()
                elif line.startswith("physical id"):
                    pid = line.split(":", 1)[1].strip()
                    sockets.add(pid)
                elif line.startswith("core id"):
                    phys.add((pid, line.split(":", 1)[1].strip()))
    except OSError:
        pass
    return {"value": rows_done / elapsed, "unit": "query-tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model, "nproc": os.cpu_count(),
            "sockets": len(sockets) or None, "physical_cores": len(phys) or None,
            "sample": f"{rows_done} query rows ({len(sample)} whole requests), every layer of "
                      f"the step, fp64 numpy oracle; {elapsed:.1f} s of compute"}


def time_layouts(case, run, dev: str, reps: int = 10):
    """Side measurements on the workload's first layer, outside the step: the same sparse
    MLA over a bf16 1,152-byte-row copy of the latent cache and over a plain-E4M3 576-byte-row
    copy with FP8 queries (same selections), and sliding-window MLA (2,048 positions) over
    the fp8 cache.  Work per launch as for the step's MLA: FLOPs 2 H (1024 + rope) per
    (row, key), bytes per selected row."""
    import torch

    from sparse_attention_decode_dsa_amd import ml4dsa as M
    from sparse_attention_decode_dsa_amd import synth
    d = case.layers[0]
    l = d["layer"]
    b = case.batch
    H, rope, K = case.mla_heads, d["rope_dim"], d["top_k"]
    li = case.inputs[l]
    nb, bs = li.lat_pool.shape[0], li.lat_pool.shape[1]
    pool16 = synth.make_latent_pool(77, nb, bs, "bf16", device=dev)
    c16 = M.make_cache(pool16, M.ML4_LAT_BF16_1152)
    pool8, kv_scale = synth.make_plain_e4m3_pool(78, nb, bs, device=dev)
    c8 = M.make_cache(pool8, M.ML4_LAT_E4M3_576)
    q8, q8s = synth.make_mla_query_fp8(79, b.total_q, H, rope, device=dev)
    idx, ln = run.topk_of(l)
    out = torch.empty((b.total_q, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b.total_q, H), dtype=torch.float32, device=dev)
    wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, run.seqs, H, K)
    ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=dev)
    fault = torch.zeros(1, dtype=torch.int32, device=dev)
    qpos = b.q_pos.cpu()
    nsel = int(ln.clamp(min=0).sum().item())
    nwin = int(torch.clamp(qpos + 1, max=K).sum().item())
    res = {}
    for name, fn, nkeys, row_b in (
            ("bf16_rows_sparse", lambda: M.ml4_sparse_mla_decode(
                run.seqs, c16, li.q_mla, M.ML4_BF16, H, rope, idx, ln, K, d["softmax_scale"],
                d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault), nsel,
             1152 if rope else 1024),
            ("e4m3_rows_sparse", lambda: M.ml4_sparse_mla_decode_e4m3(
                run.seqs, c8, kv_scale, q8, q8s, H, rope, idx, ln, K, d["softmax_scale"],
                d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault), nsel,
             576 if rope else 528),
            ("window2048_fp8", lambda: M.ml4_window_mla_decode(
                run.seqs, run.lat_caches[l], li.q_mla, M.ML4_BF16, H, rope, K,
                d["softmax_scale"], d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault), nwin,
             656 if rope else 528)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        flops = 2.0 * H * (1024 + rope) * nkeys
        res[name] = {"us": us, "TFLOPs": flops / (us * 1e-6) / 1e12,
                     "frac_f16_peak": flops / (us * 1e-6) / 1e12 / PEAK_F16_TFLOPS,
                     "row_bytes": row_b, "GBps_rows": nkeys * row_b / (us * 1e-6) / 1e9}
    assert M.ml4_fault_query(fault) == 0
    del pool16, pool8, q8, q8s
    return res


def time_cache_writes(n: int, dev: str, reps: int = 10):
    """Quantise-and-pack of n new bf16 tokens into the caches (scattered slots).  Bytes per
    token: index 128 x 2 in + 8 slot + 132 out; latent 512 x 2 + 64 x 2 in + 8 + 656 out;
    second layouts the same reads + 1,152 (bf16 rows) or 576 (plain E4M3 rows) out."""
    import torch

    from sparse_attention_decode_dsa_amd import ml4dsa as M
    g = torch.Generator(device=dev).manual_seed(1234)
    bs = 64
    nb = (n + bs - 1) // bs
    k = torch.randn(n, 128, device=dev, generator=g).to(torch.bfloat16)
    c = torch.randn(n, 512, device=dev, generator=g).to(torch.bfloat16)
    kr = torch.randn(n, 64, device=dev, generator=g).to(torch.bfloat16)
    slots = torch.randperm(nb * bs, device=dev, generator=g)[:n].to(torch.int64)
    ipool = torch.empty((nb, bs, 132), dtype=torch.uint8, device=dev)
    lpool = torch.empty((nb, bs, 656), dtype=torch.uint8, device=dev)
    bpool = torch.empty((nb, bs, 1152), dtype=torch.uint8, device=dev)
    epool = torch.empty((nb, bs, 576), dtype=torch.uint8, device=dev)
    fault = torch.zeros(1, dtype=torch.int32, device=dev)
    ic, lc = M.make_cache(ipool, M.ML4_IDX_FP8_132), M.make_cache(lpool, M.ML4_LAT_FP8_656)
    bc, ec = M.make_cache(bpool, M.ML4_LAT_BF16_1152), M.make_cache(epool, M.ML4_LAT_E4M3_576)
    out = {"tokens": n}
    for name, fn, per_tok in (
            ("index", lambda: M.ml4_index_cache_write(ic, bs, k, M.ML4_BF16, n, slots, fault), 396),
            ("latent", lambda: M.ml4_latent_cache_write(lc, bs, c, M.ML4_BF16, kr, 64, n, slots,
                                                        fault), 1816),
            ("latent_bf16_rows", lambda: M.ml4_latent_cache_write(
                bc, bs, c, M.ML4_BF16, kr, 64, n, slots, fault), 2312),
            ("latent_e4m3_rows", lambda: M.ml4_latent_cache_write_e4m3(
                ec, bs, c, M.ML4_BF16, kr, 64, 0.01, n, slots, fault), 1736)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        out[name] = {"us": us, "bytes": per_tok * n, "GBps": per_tok * n / (us * 1e-6) / 1e9}
    assert M.ml4_fault_query(fault) == 0
    return out


def time_graph_step(run, K: int):
    """The whole step through the fused entry, eager and captured into one HIP graph, K steps
    each; the replayed outputs must equal the eager ones bit for bit."""
    import torch

    def outputs():
        return [t.clone() for l in sorted(run.out) for t in (run.out[l], run.lse[l])] + \
               [t.clone() for l in sorted(run.topk_idx) for t in (run.topk_idx[l], run.topk_len[l])]

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    run.run_step(fused=True)
    torch.cuda.synchronize()
    ref = outputs()
    eager_ms = timed(lambda: run.run_step(fused=True))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run.run_step(fused=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run.run_step(fused=True)
    torch.cuda.synchronize()
    for l in run.out:
        run.out[l].fill_(float("nan"))
    graph_ms = timed(g.replay)
    got = outputs()
    same = all(torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))
               for a, b in zip(got, ref))
    del g
    return {"ms_per_step": graph_ms, "eager_fused_ms_per_step": eager_ms,
            "bit_identical_to_eager": bool(same), "steps": K}


def achievable_peaks(dev: str):
    """Rates a plain streaming read / copy and a vendor-library GEMM reach on this GPU:
    the 'measured achievable' peaks each kernel is also compared against."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3
    from sparse_attention_decode_dsa_amd import ml4dsa as M
    out = {}
    n = 1 << 31                                       # 2 GiB
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    sink = torch.zeros(8192, dtype=torch.float32, device=dev)
    t = timed(lambda: M.ml4_probe_read(x, n, sink), 5)
    out["hbm_read_GBps"] = n / t / 1e9               # the library's streaming-read probe
    t = timed(lambda: y.copy_(x), 5)
    out["hbm_copy_GBps"] = 2 * n / t / 1e9           # torch copy: read + write
    del x, y
    iters = 2000
    nwave = 256 * 8 * 4 * 4
    t = timed(lambda: M.ml4_probe_mfma(0, iters, sink), 3)
    out["mfma_f16_TFLOPs"] = nwave * 16 * iters * 16384 / t / 1e12
    t = timed(lambda: M.ml4_probe_mfma(1, iters // 2, sink), 3)
    out["mfma_fp8_TFLOPs"] = nwave * 16 * (iters // 2) * 65536 / t / 1e12
    m = 8192
    for name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        a = torch.randn(m, m, device=dev).to(dt)
        b = torch.randn(m, m, device=dev).to(dt)
        t = timed(lambda: torch.matmul(a, b), 10)
        out[f"gemm_{name}_TFLOPs"] = 2 * m ** 3 / t / 1e12
        del a, b
    try:
        a = torch.randn(m, m, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn(m, m, device=dev).to(torch.float8_e4m3fn).t()
        one = torch.ones((), device=dev)
        t = timed(lambda: torch._scaled_mm(a, b, scale_a=one, scale_b=one,
                                           out_dtype=torch.bfloat16), 10)
        out["gemm_fp8_TFLOPs"] = 2 * m ** 3 / t / 1e12
        del a, b
    except Exception as e:            # not every torch build offers an fp8 GEMM here
        out["gemm_fp8_TFLOPs"] = None
        out["gemm_fp8_note"] = f"unavailable: {type(e).__name__}"
    out["method"] = ("streaming-read probe over 2 GiB; torch copy_ of 2 GiB (read + "
                     "write); MFMA probes: 16 independent chains per wave, 8 waves per SIMD; "
                     "library GEMMs torch.matmul / _scaled_mm at 8192^3")
    return out


def mla_two_groups(rows, heads, top_k):
    """Whether the library runs fp8_ds_mla rows in its 64-head (two wave group) form: at
    most 64 heads, or when 128-head work-groups, split over keys (>= 4 tiles of 32 keys per
    split, splits doubled while the grid is under 256 work-groups), would still number
    under 256.  Mirrors the library's dispatch; used to name the kernel in reports."""
    if heads <= 64:
        return True
    groups = (heads + 127) // 128
    max_split = max(1, (top_k + 127) // 128)
    ns = 1
    while ns < max_split and rows * groups * ns < 256:
        ns <<= 1
    ns = min(ns, max_split)
    return rows * groups * ns < 256


def kernel_report(work, per, layers, case, T, ach):
    """Each kernel of each layer against its floors: HBM bytes at 8 TB/s, FP8 FLOPs at
    5.0 and 16-bit FLOPs at 2.5 PFLOP/s (datasheet), and the same against the measured
    achievable rates.  'binding' is the larger floor of the design the pages describe
    (FP8 indexer, BF16 attention); 'impl' the larger floor of the arithmetic this library
    uses (fp16 MFMA for both)."""
    rep = {}
    hbm_a = ach.get("hbm_read_GBps") or PEAK_HBM_GBS
    f16_a = ach.get("mfma_f16_TFLOPs") or PEAK_F16_TFLOPS
    fp8_a = ach.get("mfma_fp8_TFLOPs") or PEAK_FP8_TFLOPS
    for l in layers:
        w, pl = work[l], per[l]
        ent = {}
        for kern, us, nbytes, flops in (
                ("indexer", pl["indexer_us"], w["idx_bytes"], w["idx_flops"]),
                ("topk", pl["topk_us"], w["score_bytes"], 0),
                ("mla", pl["mla_us"], w["mla_bytes"], w["mla_flops"])):
            if us <= 0:
                continue
            hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e6
            fp8 = flops / (PEAK_FP8_TFLOPS * 1e12) * 1e6
            f16 = flops / (PEAK_F16_TFLOPS * 1e12) * 1e6
            binding = max(hbm, fp8 if kern == "indexer" else f16)
            impl = max(hbm, f16)
            ach_floor = max(nbytes / (hbm_a * 1e9) * 1e6, flops / (f16_a * 1e12) * 1e6)
            ent[kern] = {"us": us, "bytes": nbytes, "flops": flops,
                         "floor_us": {"hbm": hbm, "fp8": fp8, "fp16": f16},
                         "frac_binding": binding / us, "frac_impl": impl / us,
                         "frac_achievable": ach_floor / us,
                         "GBps": nbytes / (us * 1e-6) / 1e9,
                         "TFLOPs": flops / (us * 1e-6) / 1e12}
            if kern == "indexer" and flops:
                ent[kern]["frac_fp8_achievable"] = flops / (fp8_a * 1e12) * 1e6 / us
        rep[str(l)] = ent
    return rep


def time_mla_heads(case, run, dev: str, reps: int = 10):
    """Sparse MLA of the workload's first layer at 64 and 16 query heads (the pages' model
    has 64; a four-way tensor-parallel share is 16) on the same selections: the regime where
    the gather of 656-byte rows, not the matrix cores, bounds the kernel."""
    import torch

    from sparse_attention_decode_dsa_amd import ml4dsa as M
    d = case.layers[0]
    l = d["layer"]
    b = case.batch
    rope, K = d["rope_dim"], d["top_k"]
    li = case.inputs[l]
    idx, ln = run.topk_of(l)
    nsel = int(ln.clamp(min=0).sum().item())
    fault = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros(8192, dtype=torch.float32, device=dev)
    res = {}
    for H in (64, 16):
        q = li.q_mla[:, :H].contiguous()
        out = torch.empty((b.total_q, H, 512), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b.total_q, H), dtype=torch.float32, device=dev)
        wsn = M.ml4_workspace_bytes(M.ML4_ENTRY_MLA, run.seqs, H, K)
        ws = torch.empty(max(wsn, 256), dtype=torch.uint8, device=dev)
        fn = lambda: M.ml4_sparse_mla_decode(run.seqs, run.lat_pool_of(l), q, M.ML4_BF16, H,
                                             rope, idx, ln, K, d["softmax_scale"],
                                             d["ssmax_s"], out, M.ML4_BF16, lse, ws, wsn, fault)
        fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs:       # each call after the same clean 1 GiB eviction as the steps
            if M.ml4_probe_read(flush, flush.numel() * 4, flush_sink) != 0:
                raise RuntimeError(M.ml4_last_error())
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        us = 1e3 * sum(e[0].elapsed_time(e[1]) for e in evs) / reps
        row = 656 if rope else 528
        nbytes = nsel * row + b.total_q * H * ((512 + rope) * 2 + 512 * 2)
        flops = 2.0 * H * (1024 + rope) * nsel
        res[f"heads_{H}"] = {"us": us, "bytes": nbytes, "GBps": nbytes / (us * 1e-6) / 1e9,
                             "frac_hbm_peak": nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                             "TFLOPs": flops / (us * 1e-6) / 1e12,
                             "frac_f16_peak": flops / (us * 1e-6) / 1e12 / PEAK_F16_TFLOPS}
    assert M.ml4_fault_query(fault) == 0
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (one process, no collectives); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from sparse_attention_decode_dsa_amd import ml4dsa  # noqa: F401 (fails loudly if unbuilt)
    from sparse_attention_decode_dsa_amd import synth
    from sparse_attention_decode_dsa_amd.runner import CaseRunner

    torch.cuda.set_device(0)
    dev = "cuda:0"
    print(f"[bench] generating workload {args.config} on {dev}", file=sys.stderr, flush=True)
    case = synth.config(args.config, device=dev)
    torch.cuda.synchronize()
    run = CaseRunner(case)
    layers = [d["layer"] for d in case.layers]
    print(f"[bench] {case.name}: rows {case.batch.total_q}, max context "
          f"{case.batch.max_seq_len}, layers {layers}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        run.run_step(fused=args.fused)
    torch.cuda.synchronize()
    assert run.fault_bits() == 0, "fault word set during warm-up"

    K = args.steps
    # Timed region: K steps.  Before each step, outside its events, a streaming read of a
    # 1 GiB buffer (written once, here) evicts the 256 MB memory-side cache (MALL) and the
    # L2s, so every step reads its caches from HBM (the small decode workloads would
    # otherwise fit in the MALL).  The eviction is a read, not a fill: a fill leaves the
    # caches full of dirty lines whose write-back then competes with the step's own reads
    # (measured: a 138 MB read after a 1 GiB fill runs at 2.3 TB/s, after a 1 GiB read at
    # 4.8 TB/s).  Each step is bracketed by its own events; per-kernel events sit on the
    # launch stream inside the step.
    from sparse_attention_decode_dsa_amd import ml4dsa as M
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush_sink = torch.zeros(8192, dtype=torch.float32, device=dev)
    ev = {l: [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
          for l in layers}
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        if M.ml4_probe_read(flush, flush.numel() * 4, flush_sink) != 0:
            raise RuntimeError(M.ml4_last_error())
        sev[k][0].record()
        for l in layers:
            if args.fused:
                run.run_layer_fused(l)
            else:
                run.run_layer_split(l, events=ev[l][k])
        sev[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sorted(sev[k][0].elapsed_time(sev[k][1]) for k in range(K))
    ms = sum(step_ms) / K
    pct = lambda q: step_ms[min(K - 1, int(round(q * (K - 1))))]
    assert run.fault_bits() == 0, "fault word set during timing"
    # The same steps back to back, no eviction in between (caches warm where they fit).
    hot = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    hot[0].record()
    for k in range(K):
        run.run_step(fused=args.fused)
    hot[1].record()
    torch.cuda.synchronize()
    hot_ms = hot[0].elapsed_time(hot[1]) / K
    del flush, flush_sink

    work = algorithmic_work(case)
    T = case.batch.total_q
    per = {}
    if not args.fused:
        for l in layers:
            d = [x for x in case.layers if x["layer"] == l][0]
            own = d["topk_source_layer"] < 0
            per[l] = {
                "indexer_us": 1e3 * sum(ev[l][k][0].elapsed_time(ev[l][k][1]) for k in range(K)) / K if own else 0.0,
                "topk_us": 1e3 * sum(ev[l][k][1].elapsed_time(ev[l][k][2]) for k in range(K)) / K if own else 0.0,
                "mla_us": 1e3 * sum(ev[l][k][2].elapsed_time(ev[l][k][3]) for k in range(K)) / K,
            }
    step_bytes = sum(w["idx_bytes"] + w["mla_bytes"] for w in work.values())
    score_bytes = sum(w["score_bytes"] for w in work.values())
    result = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {
            "workload": case.name,
            "batch": case.batch.batch, "query_rows": T, "context": case.batch.max_seq_len,
            "block_size": case.batch.block_size, "indexer_heads": case.idx_heads,
            "mla_heads": case.mla_heads, "top_k": case.layers[0]["top_k"],
            "layers_per_step": len(layers),
            "layer_modes": [{k: d[k] for k in ("layer", "rope_dim", "kv_sharing_target_layer",
                                                "topk_source_layer", "ssmax_s")}
                            for d in case.layers],
            "us_per_layer_step": 1e3 * ms / len(layers),
            "step_ms_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
            "timing": "each step after a 1 GiB streaming read that evicts MALL/L2 with clean lines, "
                      "outside its events; "
                      "value = query rows / mean step time",
            "hot_ms_per_step": hot_ms,
            "algorithmic_bytes_per_step": step_bytes,
            "algorithmic_GBps": step_bytes / (ms * 1e-3) / 1e9,
            "score_roundtrip_bytes_per_step": score_bytes,
            "per_layer_us": per,
            "wall_s": wall,
        },
    }
    if per:
        # dominant kernel: the largest summed device time over the step
        tot = {"indexer": sum(p["indexer_us"] for p in per.values()),
               "topk": sum(p["topk_us"] for p in per.values()),
               "mla": sum(p["mla_us"] for p in per.values())}
        dom = max(tot, key=tot.get)
        l0 = layers[0]
        rope0 = case.layers[0]["rope_dim"]
        # The bound is the resource whose time floor is larger for this kernel's work.
        if dom == "indexer":
            us = per[l0]["indexer_us"]
            nbytes, flops = work[l0]["idx_bytes"], work[l0]["idx_flops"]
        elif dom == "mla":
            us = per[l0]["mla_us"]
            nbytes, flops = work[l0]["mla_bytes"], work[l0]["mla_flops"]
        else:
            us = per[l0]["topk_us"]
            nbytes, flops = work[l0]["score_bytes"], 0
        t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
        t_mfma = flops / (PEAK_F16_TFLOPS * 1e12)
        if t_mfma > t_hbm:
            ach = flops / (us * 1e-6) / 1e12
            roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_F16_TFLOPS,
                    "unit": "TFLOP/s", "frac": ach / PEAK_F16_TFLOPS}
        else:
            ach = nbytes / (us * 1e-6) / 1e9
            roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": ach / PEAK_HBM_GBS}
        roof["algorithmic_bytes"] = nbytes
        roof["algorithmic_flops"] = flops
        if case.fmt == "f32":
            roof["kernel"] = {"indexer": "k_indexer_f32", "mla": "k_mla_f32",
                              "topk": "k_topk_cand"}[dom]
        else:
            # k_mla_fp8<rope, format, two wave groups>
            tg = mla_two_groups(T, case.mla_heads, case.layers[0]["top_k"])
            roof["kernel"] = {"indexer": "k_indexer_fp8",
                              "mla": "k_mla_fp8<%d, 0, %s>" % (rope0, "true" if tg else "false"),
                              "topk": "k_topk_cand"}[dom]
        roof["layer"] = l0
        roof["avg_launch_us"] = us
        roof["traffic"] = load_traffic(dom, case.name)
        result["roofline"] = roof
    if not args.no_graph:
        result["graph_step"] = time_graph_step(run, K)
        assert run.fault_bits() == 0, "fault word set during the graph measurement"
    if not args.no_layouts and case.fmt == "fp8":
        result["layouts"] = time_layouts(case, run, dev)
        result["mla_heads"] = time_mla_heads(case, run, dev)
    if not args.no_peaks:
        print("[bench] measuring achievable peaks", file=sys.stderr, flush=True)
        result["achievable_peaks"] = achievable_peaks(dev)
        if per:
            result["kernels"] = kernel_report(work, per, layers, case, T,
                                              result["achievable_peaks"])
    if args.cache_write_tokens > 0:
        result["cache_write"] = time_cache_writes(args.cache_write_tokens, dev)
    if args.cpu_seconds > 0:
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    if args.calib_copy:
        # A plain streaming kernel with a name of its own (reads n bytes, writes n bytes), so
        # that its FETCH_SIZE / WRITE_SIZE dispatch can be told apart in a counter run.
        n = 1 << 30
        a = torch.zeros(n // 4, dtype=torch.int32, device=dev)
        b = torch.empty_like(a)
        torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
        result["config"]["calib_copy_bytes"] = n
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
