"""GPU parity of the Quest-style page selection against the fp64 oracle.

Summaries (page min/max) are exact, so they must match the oracle value for value.
Page choices follow the token rule: the selected page sets agree except for pages
whose bound lies within the fp32 error window of the selection threshold; the
current page is always there; integer inputs make every bound exact in fp32, so
the sets must then match strictly, ties included.  Attention over the GPU's token
list is compared with the oracle's attention over the same list.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import bf16_round, random_case
from parity import check_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi


def _bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _pages_of(tokens):
    """Selected pages of each row of a token list (tokens // 16 of the listed tokens)."""
    B, H, _ = tokens.shape
    return [[sorted(set((tokens[b, h][tokens[b, h] >= 0] // 16).tolist())) for h in range(H)] for b in range(B)]


def check_quest(dev, cache, q, m_per_seq, m_max, strict=False, tag=""):
    print(f"[case] {tag} B={cache.batch} N={list(cache.sl)[:6]} m={list(m_per_seq)[:6]} m_max={m_max}", flush=True)
    summ_t, summ_bits, gtok = dev.quest(m_per_seq, m_max)
    compare_quest(summ_bits, gtok, cache, q, m_per_seq, m_max, strict, tag)
    out = dev.attend(gtok)
    check_close(out, oracle.attend(cache, q, gtok), what=f"{tag} attend(quest tokens)")
    return gtok, out


def compare_quest(summ_bits, gtok, cache, q, m_per_seq, m_max, strict=False, tag=""):
    """GPU summaries (by physical page) and token lists of the sequences in `cache`
    against the oracle."""
    sm = oracle.quest_summaries(cache)
    for b in range(cache.batch):
        for p in range(-(-int(cache.sl[b]) // 16)):
            phys = int(cache.pt[b, p])
            # only pages a sequence reaches are written; the rest of the buffer is never read
            vals = _bf16_values(summ_bits[phys])
            assert np.array_equal(vals, sm[b, p]), f"{tag}: summary of page {p} of sequence {b}"
    u = oracle.quest_bounds(sm, cache.sl, q)
    opages, otok, thr = oracle.quest_select(u, cache.sl, m_per_seq, m_max)
    gpages = _pages_of(gtok)
    qf = _bf16_values(np.asarray(q))
    for b in range(cache.batch):
        n = int(cache.sl[b])
        P = -(-n // 16)
        for h in range(q.shape[1]):
            want = [p for p in opages[b, h].tolist() if p >= 0]
            got = gpages[b][h]
            assert len(got) == len(want), f"{tag}: b={b} h={h} took {len(got)} pages, want {len(want)}"
            if want:
                assert P - 1 in got, f"{tag}: b={b} h={h} lost the current page"
            # entries of a selected page: its tokens below N_b in order, -1 past N_b
            for i, p in enumerate(got):
                row = gtok[b, h, 16 * i:16 * i + 16]
                exp = np.array([16 * p + r if 16 * p + r < n else -1 for r in range(16)])
                assert np.array_equal(row, exp)
            assert np.all(gtok[b, h, 16 * len(got):] == -1)
            diff = set(got) ^ set(want)
            if strict:
                assert not diff, f"{tag}: b={b} h={h} pages differ: {sorted(diff)}"
            elif diff:
                g = h // (q.shape[1] // cache.num_kv_heads)
                ext = np.maximum(np.abs(sm[b, :P, g, 0]), np.abs(sm[b, :P, g, 1]))
                err = 2.0 ** -24 * 160 * (np.abs(qf[b, h]) * ext).sum(axis=1)    # fp32 sum bound per page
                for p in diff:
                    assert abs(u[b, h, p] - thr[b, h]) <= 2 * err.max(), \
                        f"{tag}: b={b} h={h} page {p} bound {u[b, h, p]} vs threshold {thr[b, h]}"


@pytest.mark.parametrize("cfg,kw,m", [
    (2, dict(n=4100, batch=2), 41),
    (5, dict(n=6000, batch=6, steps=1), 24),
    (3, dict(n=3001, batch=2), 10),
], ids=["C2-small", "C5-small-ragged", "C3-small"])
def test_quest_configs(cfg, kw, m):
    wl = synth.config(cfg, **kw)
    dev = DeviceCase.of_workload(wl)
    m_per_seq = np.full(wl.batch, m, np.int32)
    check_quest(dev, oracle.Cache.of(wl), wl.q, m_per_seq, m, tag=f"C{cfg}-quest")


def test_quest_long_rows_few_rows():
    """Fewer rows than CUs with page lists of 4096 pages or more take the wide page
    selection (twice the threads per row): the long-retrieval shape with 2 sequences."""
    wl = synth.config(3, n=70000, batch=2)
    dev = DeviceCase.of_workload(wl)
    m_per_seq = np.array([300, 87], np.int32)
    check_quest(dev, oracle.Cache.of(wl), wl.q, m_per_seq, 300, tag="C3-long-quest")


def test_quest_integer_strict_and_edges():
    """Integer inputs: exact bounds, many ties (lower page first); budgets of 0, 1,
    a ragged middle and more than the row holds."""
    rng = np.random.default_rng(41)
    case = random_case(rng, batch=5, hq=8, hkv=2, lens=[1, 15, 16, 700, 333], layout="fragmented",
                       integer=True, lo=-1, hi=1)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    check_quest(dev, cache, case.q, np.array([3, 0, 1, 9, 100], np.int32), 30, strict=True, tag="quest-int")


def test_quest_all_pages_is_dense_and_current_page_update():
    """A budget of every page lists every token, so attention equals dense decode
    (checked against the oracle's dense attention at fp32 accuracy: the GPU dense
    kernel rounds its softmax weights to bf16 for the MFMA and is compared at the
    usual bound elsewhere); after one appended token, re-summarising only the current
    pages equals a full re-summary."""
    rng = np.random.default_rng(42)
    case = random_case(rng, batch=3, hq=8, hkv=2, lens=[40, 161, 95], layout="shuffled")
    dev = DeviceCase.of_tiny(case)
    _, _, tok = dev.quest(np.array([50, 50, 50], np.int32), 16)
    out = dev.attend(tok)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    check_close(out, oracle.dense(cache, case.q), what="quest all pages vs dense", rtol=1e-4, atol=1e-5)
    check_close(dev.dense(), oracle.dense(cache, case.q), what="dense")
    # the tokens at N_b join the current pages (a slot of a page already in the table)
    n = case.lens.copy()
    pages = case.page_table[np.arange(3), n // 16]
    slots = n % 16
    kr = bf16_round(rng.standard_normal((3, 2, 128)))
    from device import bf16_tensor
    from helpers import bf16_bits
    dev.k[torch.from_numpy(pages).cuda(), :, torch.from_numpy(slots).cuda(), :] = bf16_tensor(bf16_bits(kr))
    dev.sl += 1
    dev.kv.n_max = int(n.max()) + 1
    # pages no sequence reaches are never written: compare the pages in use
    used = torch.from_numpy(np.concatenate([case.page_table[b, :-(-(int(n[b]) + 1) // 16)]
                                            for b in range(3)]).astype(np.int64)).cuda()
    same = lambda a, b: torch.equal(a.view(torch.int16)[used], b.view(torch.int16)[used])
    summ = sdi.quest_summarize(dev.kv)                             # full
    inc = summ.clone()
    sdi.quest_summarize(dev.kv, inc, current_pages_only=True)      # same content: idempotent
    torch.cuda.synchronize()
    assert same(summ, inc)
    # a stale summary (taken before the append) refreshed on the current pages only
    dev.sl -= 1
    dev.kv.n_max = int(n.max())
    stale = sdi.quest_summarize(dev.kv)
    dev.sl += 1
    dev.kv.n_max = int(n.max()) + 1
    torch.cuda.synchronize()
    assert not same(stale, summ)                                   # the appended rows changed a bound
    sdi.quest_summarize(dev.kv, stale, current_pages_only=True)
    torch.cuda.synchronize()
    assert same(stale, summ)


def test_quest_argument_errors():
    rng = np.random.default_rng(43)
    case = random_case(rng, batch=1, hq=4, hkv=1, lens=[20])
    dev = DeviceCase.of_tiny(case)
    summ = sdi.quest_summarize(dev.kv)
    with pytest.raises(sdi.SparseDecodeError):
        sdi.quest_select(dev.kv, dev.q, summ, i32_tensor([1]), 0)
