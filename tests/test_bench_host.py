"""Host-side checks of the benchmark's byte model (no GPU)."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden", "decode_kv_bytes_eq7.txt")


def _rows():
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            yield [int(x) for x in line.split()]


def test_dense_bytes_match_eq7():
    # dense decode must read every K and V row once per (b, kv head): the Eq. 7 figure
    # at density 1; q and out are the only other algorithmic bytes.
    rows = list(_rows())
    assert len(rows) == 4
    for batch, hkv, n, kv_bytes in rows:
        hq = 4 * hkv
        seq = np.full(batch, n)
        kps = np.full(batch, max(1, n // 50))
        _, _, dense = bench.algorithmic_bytes(seq, kps, batch, hq, hkv)
        assert dense - batch * hq * 128 * (2 + 4) == kv_bytes


def test_sparse_bytes_per_query_head():
    # per-query-head selection: each of the Hq heads reads its own k rows of K and V
    # (Eq. 7 with density G k / N per kv head) plus one 4-byte index per row
    for batch, hkv, n, kv_bytes in _rows():
        hq, k = 4 * hkv, max(1, n // 50)
        seq, kps = np.full(batch, n), np.full(batch, k)
        index, attend, _ = bench.algorithmic_bytes(seq, kps, batch, hq, hkv)
        rho = (hq // hkv) * k / n
        assert attend - batch * hq * 128 * (2 + 4) == round(kv_bytes * rho) + batch * hq * k * 4
        assert index - batch * hq * 128 * 2 - batch * hq * k * 4 == kv_bytes // 2
