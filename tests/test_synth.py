"""The seeded generator and page-table packer (no attention arithmetic involved)."""
import numpy as np
import pytest

import synth


def test_seed_reproducible_and_layout_independent():
    a = synth.make_workload("t", 5, 3, 8, 2, [40, 17, 64], synth.k_fixed(4), "contiguous")
    b = synth.make_workload("t", 5, 3, 8, 2, [40, 17, 64], synth.k_fixed(4), "shuffled")
    c = synth.make_workload("t", 5, 3, 8, 2, [40, 17, 64], synth.k_fixed(4), "fragmented")
    d = synth.make_workload("t", 6, 3, 8, 2, [40, 17, 64], synth.k_fixed(4), "shuffled")
    for bb in range(3):
        for which in "kv":
            la = a.logical_kv(which, bb)
            assert np.array_equal(la, b.logical_kv(which, bb))
            assert np.array_equal(la, c.logical_kv(which, bb))
            assert not np.array_equal(la, d.logical_kv(which, bb))
    assert np.array_equal(a.q, b.q)


def test_page_tables_are_injective_and_in_range():
    for layout in ("contiguous", "shuffled", "fragmented"):
        cap = np.array([100, 1, 16, 17, 300], dtype=np.int32)
        pt, pool = synth.make_page_table(layout, 3, cap)
        need = (cap + 15) // 16
        used = np.concatenate([pt[b, :need[b]] for b in range(len(cap))])
        assert len(np.unique(used)) == len(used)
        assert used.min() >= 0 and used.max() < pool
        if layout == "fragmented":
            assert pool == int(np.ceil(1.25 * need.sum()))


def test_growth_rows_match_a_fresh_fill():
    wl = synth.make_workload("g", 9, 2, 4, 2, [15, 33], synth.k_fixed(3), "fragmented", growth=20)
    for _ in range(20):
        wl.advance()
    fresh = synth.make_workload("g", 9, 2, 4, 2, [35, 53], synth.k_fixed(3), "contiguous")
    for b in range(2):
        for which in "kv":
            assert np.array_equal(wl.logical_kv(which, b), fresh.logical_kv(which, b))
    assert np.array_equal(wl.q, synth.queries(9, 20, 2, 4))


def test_normal_statistics():
    x = synth.bf16_to_f32(synth.queries(1, 0, 64, 64)).astype(np.float64).ravel()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    # Box-Muller tail sanity: about 4.55% beyond 2 sigma
    assert abs(np.mean(np.abs(x) > 2) - 0.0455) < 0.003


def test_outlier_channels_heavy_tailed():
    wl = synth.config(3, n=2048, batch=1)
    k = synth.bf16_to_f32(wl.logical_kv("k", 0)).astype(np.float64)
    for g in range(wl.num_kv_heads):
        ch = np.nonzero(wl.outlier_mask[0, g])[0]
        assert len(ch) == 8
        rest = np.setdiff1d(np.arange(128), ch)
        kurt = lambda v: np.mean((v - v.mean()) ** 4) / np.var(v) ** 2
        assert kurt(k[g][:, ch].ravel()) > 6.0            # t3 has infinite kurtosis
        assert abs(kurt(k[g][:, rest].ravel()) - 3.0) < 0.3


def test_planted_keys_score_high():
    wl = synth.config(2, n=2048, batch=2)
    q = synth.bf16_to_f32(wl.q).astype(np.float64)
    for b in range(2):
        k = synth.bf16_to_f32(wl.logical_kv("k", b)).astype(np.float64)
        for g in range(wl.num_kv_heads):
            pos = wl.meta["planted_positions"][(b, g)]
            assert len(pos) == 64 and len(np.unique(pos)) == 64
            for h in range(g * 4, g * 4 + 4):
                s = k[g] @ q[b, h]
                assert s[pos].min() > 30 and np.median(np.delete(s, pos)) < 5


def test_k_rules_match_printed_values():
    r = synth.k_half_up(50)
    assert r(4096) == 82 and r(32768) == 655 and r(131072) == 2621
    assert synth.k_half_up(100)(131072) == 1311 and synth.k_half_up(20)(131072) == 6554
    assert synth.k_ceil(50)(8192) == 164 and synth.k_ceil(50)(163840) == 3277 and synth.k_ceil(50)(163841) == 3277


def test_config5_lengths_and_fragmentation():
    wl = synth.config(5, n=4000, batch=8, steps=5)
    assert wl.seq_lens.min() >= 200 and wl.seq_lens.max() <= 4000
    assert np.array_equal(wl.k_per_seq(), (wl.seq_lens + 49) // 50)
    assert wl.num_pages >= int(np.ceil(1.25 * ((wl.capacity + 15) // 16).sum()))


def test_generator_sanity_against_the_oracle():
    """Not a parity check: the planted keys land in every head's exact top-k, and for
    N(0,1) data the k-th raw score sits near sqrt(128) * Phi^-1(1 - k/N)."""
    import oracle
    from statistics import NormalDist
    wl = synth.config(2, n=8192, batch=2)
    c = oracle.Cache.of(wl)
    idx, kth, _, _ = oracle.decode_step(c, wl.q, wl.k_per_seq(), wl.k_max())
    for b in range(2):
        for h in range(32):
            assert set(wl.meta["planted_positions"][(b, h // 4)]) <= set(idx[b, h].tolist())
    wl1 = synth.config(1, n=8192)
    s = oracle.scores(oracle.Cache.of(wl1), wl1.q)
    _, kth1 = oracle.topk(s, wl1.seq_lens, wl1.k_per_seq(), wl1.k_max())
    want = 128 ** 0.5 * NormalDist().inv_cdf(1 - 164 / 8192)
    assert np.all(np.abs(kth1 - want) < 3.0), (kth1, want)
