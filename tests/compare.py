"""Comparison rules between the HIP path and the CPU oracle.

Top-k sets: bit-exact, except that a position in the symmetric difference of the two sets
is accepted (and logged) when its oracle score lies within 1e-6 * max(1, |s_k|) of the
oracle's k-th score s_k (a near-tie the fp32 kernel may order differently).  Every GPU row
must also have topk_len = min(k, p+1), ascending distinct positions in [0, p] and -1
padding.  Attention: elementwise |gpu - ref| <= 2e-3 + 1e-2 |ref| on o and lse.
"""

import numpy as np
import torch

import oracle as O

TIE_REL = 1e-6
ATOL, RTOL = 2e-3, 1e-2


def batch_np(batch) -> O.Seqs:
    return O.Seqs(batch.seq_lens.cpu().numpy().astype(np.int64),
                  batch.q_start.cpu().numpy().astype(np.int64),
                  batch.q_pos.cpu().numpy().astype(np.int64),
                  batch.block_table.cpu().numpy().astype(np.int64), batch.block_size)


def t_np(t):
    """Host numpy copy; bf16 tensors come back as their uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_topk_rows(gpu_idx, gpu_len, ref_scores, q_pos, top_k, rows=None):
    """Returns (n_tie_exceptions, log lines); raises AssertionError on a violation.
    ref_scores[i] is the oracle score row of rows[i]."""
    rows = range(len(q_pos)) if rows is None else rows
    ties = []
    for i, r in enumerate(rows):
        p = int(q_pos[r])
        n = min(top_k, p + 1)
        ln = int(gpu_len[r])
        assert ln == n, f"row {r}: topk_len {ln} != {n}"
        g = np.asarray(gpu_idx[r][:ln], dtype=np.int64)
        assert (gpu_idx[r][ln:] == -1).all(), f"row {r}: padding is not -1"
        assert (np.diff(g) > 0).all(), f"row {r}: positions not strictly ascending"
        assert g.min() >= 0 and g.max() <= p, f"row {r}: position outside [0, {p}]"
        o_idx, o_len = O.topk_row(ref_scores[i], p, top_k)
        so = set(o_idx[:o_len].tolist())
        sg = set(g.tolist())
        diff = so ^ sg
        if not diff:
            continue
        s = np.asarray(ref_scores[i][:p + 1], dtype=np.float64)
        kth = np.sort(s)[::-1][n - 1]
        tau = TIE_REL * max(1.0, abs(kth))
        for t in sorted(diff):
            ok = abs(s[t] - kth) <= tau
            ties.append(f"row {r} t {t} score {s[t]!r} kth {kth!r} in_gpu {t in sg} ok {ok}")
            assert ok, "top-k set differs beyond the tie window: " + ties[-1]
    return len(ties), ties


def check_close(gpu, ref, what, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isinf(ref) & (gpu == ref)
    with np.errstate(invalid="ignore"):      # inf - inf where both sides are the same inf
        err = np.where(both_inf, 0.0, np.abs(gpu - ref))
    bound = atol + rtol * np.abs(ref)
    bad = ~(both_inf | (err <= bound))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside |d| <= {atol} + {rtol}|ref|;"
                             f" first at {tuple(i)}: gpu {gpu[tuple(i)]!r} ref {ref[tuple(i)]!r}")
    finite = ~np.isinf(ref)
    return float(err[finite].max()) if finite.any() else 0.0


def bf16_to_f64(bits):
    return O.decode_bf16(bits)
