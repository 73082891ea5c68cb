"""Comparison rules between the GPU library and the fp64 oracle.

Indices: each GPU row holds k' distinct in-range indices in ascending order, then
-1.  Outside a window of 1e-3 around the oracle's k'-th raw score the selected set
is unique and must match exactly; tokens within the window may be swapped (the
GPU accumulates q.K in fp32, the oracle in fp64).  With strict=True (inputs whose
fp32 scores are exact, e.g. small integers) no swap is allowed at all.

Outputs: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise.
"""
from __future__ import annotations

import numpy as np

WINDOW = 1e-3
ATOL = 2e-3
RTOL = 1e-2


def check_indices(gpu_idx, ora_idx, scores, kth, seq_lens, k_per_seq, strict=False, window=WINDOW):
    """Returns the number of window swaps; raises AssertionError on any violation."""
    gpu_idx = np.asarray(gpu_idx)
    B, H, k_max = gpu_idx.shape
    swaps = 0
    for b in range(B):
        n = int(seq_lens[b])
        kp = int(min(k_per_seq[b], n, k_max))
        for h in range(H):
            g = gpu_idx[b, h]
            sel = g[:kp]
            assert np.all(g[kp:] == -1), f"(b={b}, h={h}) padding is not -1"
            assert np.all(sel >= 0) and np.all(sel < n), f"(b={b}, h={h}) index out of range"
            assert np.all(np.diff(sel) > 0), f"(b={b}, h={h}) indices not strictly ascending"
            o = ora_idx[b, h, :kp]
            if np.array_equal(sel, o):
                continue
            assert not strict, f"(b={b}, h={h}) selection differs under exact scores"
            extra = np.setdiff1d(sel, o)
            missing = np.setdiff1d(o, sel)
            t = kth[b, h]
            bad = [j for j in np.concatenate([extra, missing]) if abs(scores[b, h, j] - t) > window]
            assert not bad, (f"(b={b}, h={h}) tokens {bad[:5]} differ but their scores "
                             f"{[scores[b, h, j] for j in bad[:5]]} are not within {window} of s_(k')={t}")
            swaps += len(extra)
    return swaps


def check_close(gpu, ora, atol=ATOL, rtol=RTOL, what="output"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    err = np.abs(gpu - ora)
    lim = atol + rtol * np.abs(ora)
    if not np.all(err <= lim):
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: |gpu - oracle| = {err[i]:.3e} > {lim[i]:.3e} at {i} "
                             f"(gpu {gpu[i]:.6f}, oracle {ora[i]:.6f}); max abs err {err.max():.3e}")
    return float(err.max()), float((err / np.maximum(np.abs(ora), 1e-30)).max())
