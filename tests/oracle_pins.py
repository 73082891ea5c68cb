"""Pins for the fp64 oracle: checks against what the definitions and mathematics fix.

Each pin takes the oracle's ctypes library handle, so the same checks can run
against builds of oracle.c with planted mistakes (tests/test_oracle_mutants.py).
None of them recomputes a result the way the oracle does:

* top-k:   brute force over every subset on tiny inputs (the unique set whose
           every member beats every non-member under score desc, index asc) and
           an independent rank count;
* scores:  exact rational arithmetic on logical (unpaged) tensors; integer
           inputs; shift invariance;
* attend:  the softmax formula without max-subtraction in 40-digit decimal
           arithmetic; uniform values; uniform keys; a one-hot key closed form;
           k = 1 returning the argmax row exactly;
* dense:   equal to attending over every index (k = N) and to the closed forms;
* layout:  identical results under contiguous, shuffled and fragmented pages;
* quest:   page min/max are attained bounds of the page's rows (box property); the
           page bound dominates every token score of its page, is tight on constant
           pages and has closed forms for one-signed queries; the page choice equals
           brute force over page subsets that hold the current page; every page
           selected gives dense attention;
* labels:  all channels (or keys vanishing off the channel set) give the full
           scores bit for bit; exact rationals on a tiny case.
* sampling: draws that enumerate the residual ranks give the set difference of the
           context and the kept set, in order, with weight 1; the ends of the 32-bit
           range give its first and last token; an empty residual, s = 0 and s > s_max;
           enumerating the residual once (weight 1) or twice (weight 1/2) gives dense
           attention; a residual of identical rows gives dense attention for any draws.
"""
from __future__ import annotations

import itertools
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

import oracle
from helpers import TinyCase, bf16_round, random_case

SCALE = oracle.DEFAULT_SCALE


def _cache(case: TinyCase) -> oracle.Cache:
    return oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens, case.num_kv_heads)


def _exact_scores(case: TinyCase):
    """Exact rational q.K per (b, h, j) from the logical tensors."""
    out = []
    G = case.group
    for b in range(case.batch):
        per_h = []
        for h in range(case.num_q_heads):
            qf = [Fraction(float(x)) for x in case.q_f[b, h]]
            rows = case.k_f[b][h // G]
            per_h.append([sum(qf[d] * Fraction(float(rows[j, d])) for d in range(128))
                          for j in range(rows.shape[0])])
        out.append(per_h)
    return out


def _brute_force_topk(s, k):
    """The unique size-k subset whose every member beats every non-member."""
    n = len(s)
    beats = lambda i, j: s[i] > s[j] or (s[i] == s[j] and i < j)
    found = [set(c) for c in itertools.combinations(range(n), k)
             if all(beats(i, j) for i in c for j in range(n) if j not in c)]
    assert len(found) == 1
    return sorted(found[0])


# ---------------------------------------------------------------------------- top-k

def pin_topk_bruteforce(lib):
    rng = np.random.default_rng(11)
    for trial in range(60):
        B, hq = 2, 3
        n = int(rng.integers(1, 10))
        lens = np.array([n, max(1, n - int(rng.integers(0, 3)))], dtype=np.int32)
        if trial % 2:
            s = rng.integers(-2, 3, size=(B, hq, n)).astype(np.float64)     # many ties
        else:
            s = rng.standard_normal((B, hq, n))
        kvec = rng.integers(0, n + 3, size=B).astype(np.int32)
        k_max = int(max(1, kvec.max()))
        if trial % 3 == 2:                       # a row narrower than k: keep the best k_max
            k_max = int(rng.integers(1, k_max + 1))
        idx, kth = oracle.topk(s, lens, kvec, k_max, lib=lib)
        for b in range(B):
            kp = int(min(kvec[b], lens[b], k_max))
            for h in range(hq):
                sl = list(s[b, h, :lens[b]])
                want = _brute_force_topk(sl, kp) if kp > 0 else []
                got = list(idx[b, h])
                assert got[:kp] == want, (trial, b, h, got, want)
                assert all(x == -1 for x in got[kp:])
                if kp > 0:
                    assert kth[b, h] == sorted(sl, reverse=True)[kp - 1]


def pin_topk_rank_count(lib):
    rng = np.random.default_rng(12)
    n = 300
    s = rng.integers(-4, 5, size=(1, 4, n)).astype(np.float64)
    s[0, 1] = rng.standard_normal(n)
    s[0, 2] = 0.0                                                      # all tied
    for k in (1, 7, 150, 299, 300, 301):
        idx, _ = oracle.topk(s, np.array([n], np.int32), np.array([k], np.int32), max(k, 1), lib=lib)
        kp = min(k, n)
        for h in range(4):
            sh = s[0, h]
            rank = np.array([np.sum((sh > sh[j]) | ((sh == sh[j]) & (np.arange(n) < j))) for j in range(n)])
            want = np.nonzero(rank < kp)[0]
            assert np.array_equal(idx[0, h, :kp], want), (k, h)


# ---------------------------------------------------------------------------- scores

def pin_scores_exact(lib):
    rng = np.random.default_rng(13)
    case = random_case(rng, batch=2, hq=6, hkv=2, lens=[5, 37], layout="shuffled")
    got = oracle.scores(_cache(case), case.q, lib=lib)
    ex = _exact_scores(case)
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            for j in range(case.lens[b]):
                e = float(ex[b][h][j])
                assert abs(got[b, h, j] - e) <= 1e-12 * max(1.0, abs(e)), (b, h, j, got[b, h, j], e)


def pin_scores_integer(lib):
    rng = np.random.default_rng(14)
    case = random_case(rng, batch=2, hq=8, hkv=2, lens=[40, 19], layout="fragmented", integer=True)
    got = oracle.scores(_cache(case), case.q, lib=lib)
    G = case.group
    for b in range(case.batch):
        for h in range(case.num_q_heads):
            qi = case.q_f[b, h].astype(np.int64)
            ki = case.k_f[b][h // G].astype(np.int64)
            want = ki @ qi
            assert np.array_equal(got[b, h, :case.lens[b]], want.astype(np.float64)), (b, h)


def pin_shift_invariance(lib):
    """Adding an integer vector u to every key shifts every score of a head by q.u:
    the selection (strict) and the softmax output are unchanged."""
    rng = np.random.default_rng(15)
    base = random_case(rng, batch=1, hq=4, hkv=1, lens=[48], integer=True)
    u = rng.integers(-3, 4, size=128).astype(np.float64)
    shifted = TinyCase([k + u[None, None, :] for k in base.k_f], base.v_f, base.q_f, seed=8)
    kvec = np.array([9], np.int32)
    s0 = oracle.scores(_cache(base), base.q, lib=lib)
    s1 = oracle.scores(_cache(shifted), shifted.q, lib=lib)
    for h in range(4):
        assert np.array_equal(s1[0, h] - s0[0, h], np.full(48, float(base.q_f[0, h] @ u)))
    i0, _ = oracle.topk(s0, base.lens, kvec, 9, lib=lib)
    i1, _ = oracle.topk(s1, shifted.lens, kvec, 9, lib=lib)
    assert np.array_equal(i0, i1)
    o0 = oracle.attend(_cache(base), base.q, i0, SCALE, lib=lib)
    o1 = oracle.attend(_cache(shifted), shifted.q, i1, SCALE, lib=lib)
    assert np.allclose(o0, o1, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------- attend

def pin_attend_decimal(lib):
    """Softmax without max-subtraction, in 40-digit decimal arithmetic."""
    getcontext().prec = 40
    rng = np.random.default_rng(16)
    case = random_case(rng, batch=2, hq=4, hkv=2, lens=[21, 34], layout="shuffled")
    k_max = 12
    idx = np.full((2, 4, k_max), -1, dtype=np.int32)
    for b in range(2):
        for h in range(4):
            m = int(rng.integers(1, k_max + 1))
            sel = np.sort(rng.choice(case.lens[b], size=m, replace=False))
            slots = np.sort(rng.choice(k_max, size=m, replace=False))   # -1 holes anywhere
            idx[b, h, slots] = sel
    got = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
    ex = _exact_scores(case)
    sc = Decimal(SCALE)
    for b in range(2):
        for h in range(4):
            sel = [int(j) for j in idx[b, h] if j >= 0]
            w = [(sc * Decimal(ex[b][h][j].numerator) / Decimal(ex[b][h][j].denominator)).exp() for j in sel]
            z = sum(w)
            g = h // case.group
            for d in range(128):
                num = sum(wi * Decimal(float(case.v_f[b][g][j, d])) for wi, j in zip(w, sel))
                want = float(num / z)
                assert abs(got[b, h, d] - want) <= 1e-12 * max(1.0, abs(want)), (b, h, d)


def pin_uniform_values(lib):
    rng = np.random.default_rng(17)
    case = random_case(rng, batch=2, hq=4, hkv=2, lens=[33, 16])
    v = [np.broadcast_to(bf16_round(rng.standard_normal((2, 1, 128))), (2, n, 128)).copy() for n in case.lens]
    uni = TinyCase(case.k_f, v, case.q_f)
    idx = np.full((2, 4, 8), -1, np.int32)
    idx[:, :, :5] = [0, 3, 4, 9, 15]
    for out in (oracle.attend(_cache(uni), uni.q, idx, SCALE, lib=lib), oracle.dense(_cache(uni), uni.q, SCALE, lib=lib)):
        for b in range(2):
            for h in range(4):
                assert np.allclose(out[b, h], v[b][h // 2][0], rtol=1e-14, atol=1e-14)


def pin_uniform_keys(lib):
    """Identical keys: every score ties, the first k' indices win, o = mean of their values."""
    rng = np.random.default_rng(18)
    n = 41
    krow = bf16_round(rng.standard_normal(128))
    k = [np.broadcast_to(krow, (1, n, 128)).copy()]
    v = [bf16_round(rng.standard_normal((1, n, 128)))]
    case = TinyCase(k, v, bf16_round(rng.standard_normal((1, 3, 128))))
    for kk in (1, 5, 40, 41, 60):
        s = oracle.scores(_cache(case), case.q, lib=lib)
        idx, _ = oracle.topk(s, case.lens, np.array([kk], np.int32), kk, lib=lib)
        kp = min(kk, n)
        for h in range(3):
            assert np.array_equal(idx[0, h, :kp], np.arange(kp))
        out = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
        want = v[0][0, :kp].mean(axis=0)
        assert np.allclose(out[0], want[None, :], rtol=1e-13, atol=1e-14)
    dense = oracle.dense(_cache(case), case.q, SCALE, lib=lib)
    assert np.allclose(dense[0], v[0][0].mean(axis=0)[None, :], rtol=1e-13, atol=1e-14)


def pin_one_hot(lib):
    """K_{j*} = c e_m, all other keys 0: S = {j*} + the first k'-1 other indices, and
    o = a V_{j*} + (1-a)/(k'-1) sum_{S minus j*} V with a = e^x / (e^x + k' - 1), x = c q_m / sqrt(128)."""
    rng = np.random.default_rng(19)
    n, m, jstar, c = 50, 17, 37, 4.0
    for sign in (1.0, -1.0):
        q = bf16_round(rng.standard_normal((1, 2, 128)))
        q[0, :, m] = sign * np.array([1.5, 0.75])
        k = np.zeros((1, 1, n, 128))
        k[0, 0, jstar, m] = c
        v = bf16_round(rng.standard_normal((1, 1, n, 128)))
        case = TinyCase([k[0]], [v[0]], q)
        for kk in (1, 6, 20):
            s = oracle.scores(_cache(case), case.q, lib=lib)
            idx, _ = oracle.topk(s, case.lens, np.array([kk], np.int32), kk, lib=lib)
            out = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
            for h in range(2):
                if sign > 0:
                    others = [j for j in range(n) if j != jstar][:kk - 1]
                    want_set = sorted([jstar] + others)
                    x = c * q[0, h, m] * SCALE
                    a = math.exp(x) / (math.exp(x) + kk - 1)
                    want_o = a * v[0, 0, jstar] + ((1 - a) / (kk - 1) * v[0, 0, others].sum(axis=0) if kk > 1 else 0)
                else:
                    want_set = list(range(kk))
                    want_o = v[0, 0, :kk].mean(axis=0)
                assert list(idx[0, h]) == want_set, (sign, kk, h)
                assert np.allclose(out[0, h], want_o, rtol=1e-12, atol=1e-13), (sign, kk, h)


def pin_k1_argmax_row(lib):
    rng = np.random.default_rng(20)
    case = random_case(rng, batch=2, hq=4, hkv=1, lens=[29, 64])
    s = oracle.scores(_cache(case), case.q, lib=lib)
    idx, _ = oracle.topk(s, case.lens, np.array([1, 1], np.int32), 1, lib=lib)
    out = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
    ex = _exact_scores(case)
    for b in range(2):
        for h in range(4):
            j = int(np.argmax([float(x) for x in ex[b][h]]))
            assert idx[0 + b, h, 0] == j
            assert np.array_equal(out[b, h], case.v_f[b][0][j])


# ---------------------------------------------------------------------------- dense / invariants

def pin_dense_is_attend_all(lib):
    rng = np.random.default_rng(21)
    case = random_case(rng, batch=3, hq=10, hkv=2, lens=[1, 17, 45], layout="fragmented")
    n_max = int(case.lens.max())
    idx = np.full((3, 10, n_max), -1, np.int32)
    for b in range(3):
        idx[b, :, :case.lens[b]] = np.arange(case.lens[b])
    d = oracle.dense(_cache(case), case.q, SCALE, lib=lib)
    a = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
    assert np.allclose(d, a, rtol=1e-12, atol=1e-14)
    s = oracle.scores(_cache(case), case.q, lib=lib)
    i2, _ = oracle.topk(np.nan_to_num(s, nan=-1e300), case.lens, case.lens, n_max, lib=lib)
    assert np.array_equal(i2, idx)                           # k >= N selects everything
    # a direct fp64 softmax on the logical tensors (max-subtracted, numpy)
    for b in range(3):
        for h in range(10):
            sc = case.k_f[b][h // 5] @ case.q_f[b, h] * SCALE
            w = np.exp(sc - sc.max())
            want = (w[:, None] * case.v_f[b][h // 5]).sum(0) / w.sum()
            assert np.allclose(d[b, h], want, rtol=1e-11, atol=1e-13)


def pin_layout_invariance(lib):
    rng = np.random.default_rng(22)
    base = random_case(rng, batch=3, hq=4, hkv=2, lens=[37, 16, 70], layout="contiguous")
    res = []
    for layout, seed in (("contiguous", 1), ("shuffled", 2), ("fragmented", 3)):
        case = TinyCase(base.k_f, base.v_f, base.q_f, layout=layout, seed=seed)
        s = oracle.scores(_cache(case), case.q, lib=lib)
        idx, kth = oracle.topk(np.nan_to_num(s, nan=0.0), case.lens, np.array([5, 16, 9], np.int32), 16, lib=lib)
        out = oracle.attend(_cache(case), case.q, idx, SCALE, lib=lib)
        dn = oracle.dense(_cache(case), case.q, SCALE, lib=lib)
        res.append((np.nan_to_num(s), idx, kth, out, dn))
    for other in res[1:]:
        for x, y in zip(res[0], other):
            assert np.array_equal(x, y)


# ---------------------------------------------------------------------------- quest pages

def _quest_case(rng, layout="fragmented"):
    return random_case(rng, batch=4, hq=6, hkv=2, lens=[1, 16, 17, 61], layout=layout)


def pin_quest_box(lib):
    """min/max of a page: every cached row lies inside, each bound is attained."""
    rng = np.random.default_rng(31)
    case = _quest_case(rng)
    sm = oracle.quest_summaries(_cache(case), lib=lib)
    for b in range(case.batch):
        n = int(case.lens[b])
        pages = -(-n // 16)
        assert np.all(np.isnan(sm[b, pages:]))
        for p in range(pages):
            for g in range(case.num_kv_heads):
                rows = case.k_f[b][g][16 * p:min(n, 16 * p + 16)]
                mn, mx = sm[b, p, g, 0], sm[b, p, g, 1]
                assert np.all(rows >= mn) and np.all(rows <= mx)
                assert np.all((rows == mn).any(axis=0)) and np.all((rows == mx).any(axis=0))


def pin_quest_bound(lib):
    """The bound dominates the page's token scores; tight on constant pages; one-signed
    queries give sum q max (q >= 0) or sum q min (q <= 0)."""
    rng = np.random.default_rng(32)
    case = _quest_case(rng, layout="shuffled")
    c = _cache(case)
    u = oracle.quest_bounds(oracle.quest_summaries(c, lib=lib), c.sl, case.q, lib=lib)
    s = oracle.scores(c, case.q, lib=lib)
    for b in range(case.batch):
        n = int(case.lens[b])
        for h in range(case.num_q_heads):
            for j in range(n):
                assert s[b, h, j] <= u[b, h, j // 16] + 1e-9 * (1 + abs(u[b, h, j // 16]))
    # constant pages: every row of a page equal -> the bound is that row's score
    k = [np.repeat(bf16_round(rng.standard_normal((2, 3, 1, 128))), 16, axis=2).reshape(2, 48, 128)]
    v = [bf16_round(rng.standard_normal((2, 48, 128)))]
    q = bf16_round(rng.standard_normal((1, 4, 128)))
    tc = TinyCase(k, v, q, layout="fragmented", seed=5)
    tcc = _cache(tc)
    u2 = oracle.quest_bounds(oracle.quest_summaries(tcc, lib=lib), tcc.sl, tc.q, lib=lib)
    s2 = oracle.scores(tcc, tc.q, lib=lib)
    assert np.allclose(u2[0, :, :3], s2[0, :, ::16], rtol=1e-13, atol=1e-12)
    # one-signed queries
    qp = np.abs(bf16_round(rng.standard_normal((1, 4, 128))))
    for sign, col in ((1.0, 1), (-1.0, 0)):
        qs = TinyCase(case.k_f[3:], case.v_f[3:], sign * qp, layout="contiguous")
        qc = _cache(qs)
        u3 = oracle.quest_bounds(oracle.quest_summaries(qc, lib=lib), qc.sl, qs.q, lib=lib)
        rows = case.k_f[3]
        for h in range(4):
            for p in range(-(-int(qs.lens[0]) // 16)):
                blk = rows[h // 2][16 * p:16 * p + 16]
                ext = blk.max(axis=0) if col == 1 else blk.min(axis=0)
                want = float(sum(Fraction(float(a)) * Fraction(float(x)) for a, x in zip(sign * qp[0, h], ext)))
                assert abs(u3[0, h, p] - want) <= 1e-12 * (1 + abs(want))


def _brute_force_pages(u, n, m):
    """The pages of a sequence of n tokens chosen under budget m by brute force: the
    current page plus the subset of the others whose every member beats every
    non-member (bound desc, page asc)."""
    P = -(-n // 16)
    m = min(m, P)
    if m <= 0:
        return []
    others = list(range(P - 1))
    beats = lambda i, j: u[i] > u[j] or (u[i] == u[j] and i < j)
    found = [set(c) for c in itertools.combinations(others, m - 1)
             if all(beats(i, j) for i in c for j in others if j not in c)]
    assert len(found) == 1
    return sorted(found[0] | {P - 1})


def pin_quest_select_bruteforce(lib):
    rng = np.random.default_rng(33)
    for trial in range(60):
        B, hq = 3, 2
        lens = rng.integers(1, 113, size=B).astype(np.int32)   # up to 8 pages
        m = rng.integers(0, 10, size=B).astype(np.int32)
        m_max = 6
        u = rng.integers(-3, 4, size=(B, hq, 8)).astype(np.float64)   # many ties
        pages, toks, thr = oracle.quest_select(u, lens, m, m_max, lib=lib)
        for b in range(B):
            for h in range(hq):
                want = _brute_force_pages(u[b, h], int(lens[b]), min(int(m[b]), m_max))
                assert pages[b, h].tolist() == want + [-1] * (m_max - len(want))
                tk = [j for p in want for j in range(16 * p, min(int(lens[b]), 16 * p + 16))]
                assert toks[b, h].tolist() == tk + [-1] * (16 * m_max - len(tk))
                ranked = [p for p in want if p != -(-int(lens[b]) // 16) - 1]
                if ranked:
                    assert thr[b, h] == min(u[b, h, p] for p in ranked)
                else:
                    assert thr[b, h] == np.inf


def pin_quest_all_pages_is_dense(lib):
    rng = np.random.default_rng(34)
    case = random_case(rng, batch=3, hq=4, hkv=2, lens=[5, 33, 64], layout="fragmented")
    c = _cache(case)
    u = oracle.quest_bounds(oracle.quest_summaries(c, lib=lib), c.sl, case.q, lib=lib)
    _, toks, _ = oracle.quest_select(u, c.sl, np.array([4, 4, 4], np.int32), 4, lib=lib)
    a = oracle.attend(c, case.q, toks, SCALE, lib=lib)
    d = oracle.dense(c, case.q, SCALE, lib=lib)
    assert np.allclose(a, d, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------- label scores

def pin_label_scores(lib):
    """All 128 channels in order give the full scores bit for bit; keys that vanish off
    a 16-channel set give the full scores too; exact rationals on a tiny case."""
    rng = np.random.default_rng(35)
    case = random_case(rng, batch=2, hq=4, hkv=2, lens=[9, 40], layout="fragmented")
    c = _cache(case)
    full = oracle.scores(c, case.q, lib=lib)
    allch = np.tile(np.arange(128, dtype=np.int32), (2, 1))
    assert np.array_equal(np.nan_to_num(oracle.label_scores(c, case.q, allch, lib=lib)), np.nan_to_num(full))
    ch = np.stack([np.sort(rng.choice(128, 16, replace=False)) for _ in range(2)]).astype(np.int32)
    k = [np.zeros_like(kf) for kf in case.k_f]
    for b in range(2):
        for g in range(2):
            k[b][g][:, ch[g]] = case.k_f[b][g][:, ch[g]]
    zc = TinyCase(k, case.v_f, case.q_f, layout="shuffled", seed=3)
    zcc = _cache(zc)
    assert np.array_equal(np.nan_to_num(oracle.label_scores(zcc, zc.q, ch, lib=lib)),
                          np.nan_to_num(oracle.scores(zcc, zc.q, lib=lib)))
    got = oracle.label_scores(c, case.q, ch, lib=lib)
    for b in range(2):
        for h in range(4):
            g = h // 2
            for j in range(int(case.lens[b])):
                want = sum(Fraction(float(case.q_f[b, h, d])) * Fraction(float(case.k_f[b][g][j, d])) for d in ch[g])
                assert abs(got[b, h, j] - float(want)) <= 1e-12 * (1 + abs(float(want)))


# ---------------------------------------------------------------------------- stochastic selection

def _enumerating_draws(M, reps=1):
    """32-bit draws whose ranks floor(x M / 2^32) are 0, 1, ..., M-1 (each reps times)."""
    ranks = [r for r in range(M) for _ in range(reps)]
    return [(r * 2 ** 32 + M - 1) // M for r in ranks]


def _kept_rows(rng, lens, hq, k_max, kvec):
    """Random kept sets in the top-k row format: ascending valid tokens, then -1."""
    B = len(lens)
    idx = np.full((B, hq, k_max), -1, np.int32)
    for b in range(B):
        kp = min(int(kvec[b]), k_max, int(lens[b]))
        for h in range(hq):
            idx[b, h, :kp] = np.sort(rng.choice(int(lens[b]), size=kp, replace=False))
    return idx


def pin_sample_enumeration(lib):
    rng = np.random.default_rng(36)
    lens = np.array([30, 7, 12, 50], np.int32)
    kvec = np.array([5, 7, 0, 9], np.int32)          # row 1 keeps everything: empty residual
    hq, k_max, s_max = 3, 10, 50
    idx = _kept_rows(rng, lens, hq, k_max, kvec)
    draws = np.zeros((4, hq, s_max), np.uint32)
    svec = np.zeros(4, np.int32)
    for b in range(4):
        M = int(lens[b]) - min(int(kvec[b]), int(lens[b]))
        svec[b] = max(M, 1)
        for h in range(hq):
            draws[b, h, :M] = _enumerating_draws(M) if M else []
    sample, weight = oracle.sample_residual(idx, kvec, lens, draws, svec, lib=lib)
    for b in range(4):
        for h in range(hq):
            kept = set(idx[b, h][idx[b, h] >= 0].tolist())
            rest = sorted(set(range(int(lens[b]))) - kept)
            M = len(rest)
            assert sample[b, h, :M].tolist() == rest, (b, h)
            assert np.all(sample[b, h, M:] == -1)
            assert weight[b, h] == (1.0 if M else 0.0)
    # the ends of the 32-bit range; s > s_max is clipped; s = 0 draws nothing
    d2 = np.zeros((4, hq, 2), np.uint32)
    d2[..., 1] = 2 ** 32 - 1
    sample, weight = oracle.sample_residual(idx, kvec, lens, d2, np.array([5, 5, 0, 2], np.int32), lib=lib)
    for b, h in itertools.product(range(4), range(hq)):
        rest = sorted(set(range(int(lens[b]))) - set(idx[b, h][idx[b, h] >= 0].tolist()))
        if b in (1, 2):
            assert sample[b, h].tolist() == [-1, -1] and weight[b, h] == 0.0
        else:
            assert sample[b, h].tolist() == [rest[0], rest[-1]] and weight[b, h] == len(rest) / 2


def pin_sampled_enumeration_is_dense(lib):
    """Every residual token drawn once (weight 1) or twice (weight 1/2): the estimate is
    the dense output."""
    rng = np.random.default_rng(37)
    case = random_case(rng, batch=3, hq=4, hkv=2, lens=[23, 40, 9], layout="fragmented")
    c = _cache(case)
    kvec = np.array([6, 11, 3], np.int32)
    idx, _ = oracle.topk(oracle.scores(c, case.q, lib=lib), c.sl, kvec, 11, lib=lib)
    dense = oracle.dense(c, case.q, SCALE, lib=lib)
    for reps in (1, 2):
        s_max = 2 * 40
        draws = np.zeros((3, 4, s_max), np.uint32)
        svec = np.zeros(3, np.int32)
        for b in range(3):
            M = int(case.lens[b]) - int(kvec[b])
            svec[b] = reps * M
            draws[b, :, :reps * M] = _enumerating_draws(M, reps)
        sample, weight = oracle.sample_residual(idx, kvec, c.sl, draws, svec, lib=lib)
        for b in range(3):
            assert np.all(weight[b] == 1.0 / reps)
        est = oracle.attend_sampled(c, case.q, idx, sample, weight, SCALE, lib=lib)
        assert np.allclose(est, dense, rtol=1e-12, atol=1e-14), reps


def pin_sampled_identical_residual(lib):
    """All tokens outside the kept set share one key row and one value row: whatever
    is drawn, M / s' copies per draw rebuild the residual's sums exactly."""
    rng = np.random.default_rng(38)
    lens = [37, 64]
    hkv, hq, k_max = 2, 4, 8
    kvec = np.array([5, 8], np.int32)
    idx = _kept_rows(rng, np.array(lens, np.int32), hq, k_max, kvec)
    k = [bf16_round(rng.standard_normal((hkv, n, 128))) for n in lens]
    v = [bf16_round(rng.standard_normal((hkv, n, 128))) for n in lens]
    for b, n in enumerate(lens):
        kept = set(idx[b, 0][idx[b, 0] >= 0].tolist())
        for h in range(1, hq):
            idx[b, h] = idx[b, 0]                     # one kept set per sequence
        krow, vrow = bf16_round(rng.standard_normal((2, hkv, 128)))
        for j in range(n):
            if j not in kept:
                k[b][:, j], v[b][:, j] = krow, vrow
    case = TinyCase(k, v, bf16_round(rng.standard_normal((2, hq, 128))), layout="shuffled")
    c = _cache(case)
    dense = oracle.dense(c, case.q, SCALE, lib=lib)
    for s in (1, 3, 7):
        draws = rng.integers(0, 2 ** 32, size=(2, hq, 7), dtype=np.uint64).astype(np.uint32)
        sample, weight = oracle.sample_residual(idx, kvec, c.sl, draws, np.array([s, s], np.int32), lib=lib)
        est = oracle.attend_sampled(c, case.q, idx, sample, weight, SCALE, lib=lib)
        assert np.allclose(est, dense, rtol=1e-12, atol=1e-14), s


ALL_PINS = [
    pin_topk_bruteforce, pin_topk_rank_count, pin_scores_exact, pin_scores_integer,
    pin_shift_invariance, pin_attend_decimal, pin_uniform_values, pin_uniform_keys, pin_one_hot,
    pin_k1_argmax_row, pin_dense_is_attend_all, pin_layout_invariance,
    pin_quest_box, pin_quest_bound, pin_quest_select_bruteforce, pin_quest_all_pages_is_dense,
    pin_label_scores,
    pin_sample_enumeration, pin_sampled_enumeration_is_dense, pin_sampled_identical_residual,
]
