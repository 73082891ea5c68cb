"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Sizes are ones the oracle finishes in seconds yet span several score chunks
(1024 tokens), several attend chunks (256 indices) and a ragged tail; the
full-size workloads are in test_gpu_full_size.py.  Comparison rules are in
tests/parity.py.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import TinyCase, bf16_round, random_case
from parity import check_close, check_indices

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi


def _say(*a):
    print(*a, flush=True)


def run_and_check(dev, cache, q, k_per_seq, k_max, strict=False, check_dense=True, tag=""):
    """Index + attend + dense on the GPU, each against the oracle.  Returns GPU results."""
    _say(f"[case] {tag} B={cache.batch} Hq={q.shape[1]} Hkv={cache.num_kv_heads} "
         f"N={list(cache.sl)[:4]} k={list(k_per_seq)[:4]} k_max={k_max}")
    s = oracle.scores(cache, q)
    ora_idx, kth = oracle.topk(np.nan_to_num(s, nan=-np.inf), cache.sl, k_per_seq, k_max)
    gpu_idx = dev.index(k_per_seq, k_max)
    swaps = check_indices(gpu_idx, ora_idx, s, kth, cache.sl, k_per_seq, strict=strict)
    # attend on the oracle's list (both sides see the same rows)
    ora_out = oracle.attend(cache, q, ora_idx)
    gpu_out = dev.attend(ora_idx, k_per_seq)
    check_close(gpu_out, ora_out, what=f"{tag} attend(oracle idx)")
    # end to end: the GPU's own (validated) list on both sides
    e2e = dev.attend(gpu_idx, k_per_seq)
    check_close(e2e, oracle.attend(cache, q, gpu_idx), what=f"{tag} attend(gpu idx)")
    dn = None
    if check_dense:
        dn = dev.dense()
        check_close(dn, oracle.dense(cache, q), what=f"{tag} dense")
    return gpu_idx, e2e, dn, swaps


# ------------------------------------------------------------------------ configurations

def test_config1_full_size():
    wl = synth.config(1)
    dev = DeviceCase.of_workload(wl)
    run_and_check(dev, oracle.Cache.of(wl), wl.q, wl.k_per_seq(), wl.k_max(), tag="C1")


@pytest.mark.parametrize("cfg,kw", [
    (2, dict(n=4100, batch=2)),
    (3, dict(n=3001, batch=2)),
    (5, dict(n=6000, batch=6, steps=1)),
], ids=["C2-small", "C3-small", "C5-small"])
def test_config_small(cfg, kw):
    wl = synth.config(cfg, **kw)
    dev = DeviceCase.of_workload(wl)
    run_and_check(dev, oracle.Cache.of(wl), wl.q, wl.k_per_seq(), wl.k_max(), tag=f"C{cfg}-small")


@pytest.mark.parametrize("cfg,kw", [
    (2, dict(n=8192, batch=32)),
    (5, dict(n=4096, batch=64, steps=1)),
], ids=["C2-B32", "C5-B64-ragged"])
def test_two_slot_workgroups(cfg, kw):
    """Grids of one or two rounds score two 512-token slots per wave (the first slot's
    flush overlapping the second's loads); these shapes take that path, the ragged one
    with waves whose second slot is partial or empty."""
    wl = synth.config(cfg, **kw)
    blocks2 = -(-wl.n_max // 4096) * wl.num_kv_heads * -(-wl.group // 8) * wl.batch
    assert 2 * 256 <= blocks2 <= 4 * 256
    dev = DeviceCase.of_workload(wl)
    run_and_check(dev, oracle.Cache.of(wl), wl.q, wl.k_per_seq(), wl.k_max(), tag=f"C{cfg}-two-slot")


@pytest.mark.parametrize("cfg,kw,ratios", [
    (4, dict(n=5000, batch=2, steps=3), (100, 50, 20, 1)),
    (5, dict(n=6000, batch=6, steps=3), (50,)),
], ids=["C4-small-sweep", "C5-small-growth"])
def test_multi_step_growth(cfg, kw, ratios):
    """Cache growth by one token per step (appended on the device with plain copies);
    every step is checked, for each sparsity ratio (k = N runs dense as well)."""
    wl = synth.config(cfg, **kw)
    dev = DeviceCase.of_workload(wl)
    for step in range(wl.steps):
        if step > 0:
            rows = wl.advance()                          # host copy for the oracle
            dev.append(rows, wl.q, wl.n_max)
        cache = oracle.Cache.of(wl)
        for r in ratios:
            rule = synth.k_ceil(r) if cfg == 5 else synth.k_half_up(r)
            kps = rule(wl.seq_lens)
            gidx, e2e, dn, _ = run_and_check(dev, cache, wl.q, kps, int(kps.max()), check_dense=(r == 1 or r == ratios[0]),
                                             tag=f"C{cfg} step{step} N/{r}")
            if r == 1:                                   # k = N: the sparse path equals dense
                check_close(e2e, dn, what="k=N sparse vs dense")


# ------------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("hq,hkv", [(3, 3), (4, 2), (16, 2), (10, 2), (32, 2), (64, 2)],
                         ids=["G1", "G2", "G8", "G5", "G16", "G32-two-head-blocks"])
def test_group_sizes(hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv)
    case = random_case(rng, batch=2, hq=hq, hkv=hkv, lens=[37, 1300], layout="shuffled")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    run_and_check(dev, cache, case.q, np.array([5, 300], np.int32), 300, tag=f"G{hq // hkv}")


@pytest.mark.parametrize("lens,kvec,k_max", [
    ([1, 5, 16, 17], [1, 1, 1, 1], 1),                  # k = 1, tiny contexts
    ([1, 5, 16, 17], [3, 9, 40, 17], 40),               # k >= N clamps to N, padding
    ([2500, 1000, 3333], [2500, 7, 999], 2600),         # k = N, ragged k
    ([4096, 2049], [4000, 2049], 4096),                 # k close to N
    ([9000], [8500], 8500),                              # k beyond the attend chunk count
    ([3000, 5, 700, 40], [0, 5, 0, 3], 64),              # k = 0 rows: all -1, attend gives 0
], ids=["k1", "k-ge-N", "ragged-k", "k-near-N", "big-k", "k0"])
def test_k_edges(lens, kvec, k_max):
    rng = np.random.default_rng(len(lens) * 7 + k_max)
    case = random_case(rng, batch=len(lens), hq=8, hkv=2, lens=lens, layout="fragmented")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    run_and_check(dev, cache, case.q, np.array(kvec, np.int32), k_max, tag="k-edge")


def test_k1_returns_argmax_row_exactly():
    rng = np.random.default_rng(5)
    case = random_case(rng, batch=2, hq=4, hkv=1, lens=[700, 2000], integer=True, lo=-3, hi=3)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    kv = np.array([1, 1], np.int32)
    gidx = dev.index(kv, 1)
    s = oracle.scores(cache, case.q)
    oidx, _ = oracle.topk(np.nan_to_num(s, nan=-np.inf), case.lens, kv, 1)
    assert np.array_equal(gidx, oidx)
    out = dev.attend(gidx, kv)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], case.v_f[b][0][gidx[b, h, 0]].astype(np.float32))


def test_integer_inputs_strict():
    """Small-integer q and K make every fp32 score exact: the selection must match
    the oracle exactly, ties included."""
    rng = np.random.default_rng(6)
    case = random_case(rng, batch=3, hq=8, hkv=2, lens=[3000, 1111, 2048], integer=True, lo=-1, hi=1)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    run_and_check(dev, cache, case.q, np.array([60, 500, 2047], np.int32), 2047, strict=True, tag="int")


def test_uniform_keys_take_first_indices():
    rng = np.random.default_rng(7)
    n = [1500, 777]
    krow = bf16_round(rng.standard_normal(128))
    k = [np.broadcast_to(krow, (2, x, 128)).copy() for x in n]
    v = [bf16_round(rng.standard_normal((2, x, 128))) for x in n]
    case = TinyCase(k, v, bf16_round(rng.standard_normal((2, 8, 128))))
    dev = DeviceCase.of_tiny(case)
    kv = np.array([300, 40], np.int32)
    gidx = dev.index(kv, 300)
    assert np.array_equal(gidx[0, :, :300], np.broadcast_to(np.arange(300), (8, 300)))
    assert np.array_equal(gidx[1, :, :40], np.broadcast_to(np.arange(40), (8, 40)))
    assert np.all(gidx[1, :, 40:] == -1)
    out = dev.attend(gidx, kv)
    check_close(out[0], np.broadcast_to(v[0][:, :300].mean(1).repeat(4, 0), (8, 128)), what="uniform keys b0")
    check_close(out[1], np.broadcast_to(v[1][:, :40].mean(1).repeat(4, 0), (8, 128)), what="uniform keys b1")


def test_one_hot_key():
    rng = np.random.default_rng(8)
    n, m, jstar, c = 3000, 40, 2222, 4.0
    q = bf16_round(rng.standard_normal((1, 4, 128)))
    q[0, :, m] = [1.5, 0.75, -1.0, 2.0]
    k = np.zeros((1, n, 128))
    k[0, jstar, m] = c
    v = bf16_round(rng.standard_normal((1, n, 128)))
    case = TinyCase([k], [v], q)
    dev = DeviceCase.of_tiny(case)
    kk = 20
    gidx = dev.index(np.array([kk], np.int32), kk)
    for h in range(4):
        want = sorted([jstar] + list(range(kk - 1))) if q[0, h, m] > 0 else list(range(kk))
        assert list(gidx[0, h]) == want, h
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    check_close(dev.attend(gidx), oracle.attend(cache, case.q, gidx), what="one-hot attend")


def test_attend_accepts_any_index_list():
    """-1 holes anywhere, out-of-range entries skipped, k_per_seq omitted."""
    rng = np.random.default_rng(9)
    case = random_case(rng, batch=2, hq=4, hkv=1, lens=[900, 3000])
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    k_max = 700
    idx = np.full((2, 4, k_max), -1, np.int32)
    for b in range(2):
        for h in range(4):
            m = int(rng.integers(0, k_max))
            idx[b, h, rng.choice(k_max, size=m, replace=False)] = rng.choice(case.lens[b], size=m, replace=False)
    idx[0, 0, :] = -1                                      # an empty row gives 0
    idx[1, 1, 5] = 5000                                    # beyond N_b: skipped
    gpu = dev.attend(idx, None)
    idx_o = np.where(idx >= case.lens[:, None, None], -1, idx)
    check_close(gpu, oracle.attend(cache, case.q, idx_o), what="holes")
    assert np.all(gpu[0, 0] == 0)


@pytest.mark.parametrize("k_max", [700, 1300], ids=["one-workgroup", "chunked"])
def test_attend_counts_cut_the_list(k_max):
    """k_per_seq limits the row to its first k_b entries even where the list holds more;
    k_b = 0 gives 0 and k_b > k_max is clamped to k_max."""
    rng = np.random.default_rng(19)
    case = random_case(rng, batch=3, hq=4, hkv=2, lens=[1500, 3000, 2000])
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    idx = np.stack([np.stack([np.sort(rng.choice(case.lens[b], size=k_max, replace=False)) for _ in range(4)])
                    for b in range(3)]).astype(np.int32)
    kps = np.array([0, 37, k_max + 500], np.int32)
    gpu = dev.attend(idx, kps)
    cut = idx.copy()
    for b in range(3):
        cut[b, :, min(kps[b], k_max):] = -1
    assert np.all(gpu[0] == 0)
    check_close(gpu[1:], oracle.attend(cache, case.q, cut)[1:], what="counts")


def test_layout_invariance_and_determinism():
    rng = np.random.default_rng(10)
    base = random_case(rng, batch=3, hq=8, hkv=2, lens=[2000, 333, 4100], layout="contiguous")
    kv = np.array([40, 333, 82], np.int32)
    res = []
    for layout, seed in (("contiguous", 1), ("shuffled", 2), ("fragmented", 3), ("shuffled", 2)):
        case = TinyCase(base.k_f, base.v_f, base.q_f, layout=layout, seed=seed)
        dev = DeviceCase.of_tiny(case)
        gidx = dev.index(kv, 333)
        res.append((gidx, dev.attend(gidx, kv), dev.dense()))
    for other in res[1:]:
        for a, b in zip(res[0], other):
            assert np.array_equal(a, b)


def test_workspace_too_small_is_rejected():
    wl = synth.config(1)
    dev = DeviceCase.of_workload(wl)
    need = sdi.index_topk_workspace_bytes(dev.kv, 4, 82)
    ws = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        sdi.index_topk(dev.kv, dev.q, i32_tensor(wl.k_per_seq()), 82, workspace=ws)


# ------------------------------------------------------------------------ long rows and select paths

def test_long_rows_many_slots():
    """Rows of more than 512 slots (262144 tokens): the select reads the slot headers in
    several passes; a 270000-token row beside a 40000-token one, fragmented pages.  The
    cache is drawn straight into its pages as bf16 bit patterns (random sign and 7-bit
    mantissa in [0.5, 1); V reuses K's bits, the other tests keep them apart)."""
    rng = np.random.default_rng(29)
    lens = np.array([270000, 40000], np.int32)
    pt, pool = synth.make_page_table("fragmented", 29, lens)

    def draw(*shape):
        return (rng.integers(0, 1 << 16, size=shape, dtype=np.uint16) & 0x807F) | 0x3F00
    k_cache, q = draw(pool, 1, 16, 128), draw(2, 4, 128)
    dev = DeviceCase(k_cache, k_cache, pt, lens, q)
    cache = oracle.Cache(k_cache, k_cache, pt, lens, 1)
    run_and_check(dev, cache, q, np.array([5400, 800], np.int32), 5400, tag="long rows")


def test_select_fallback_paths():
    """Threshold bins too large for the LDS candidate list (all keys tied; few distinct
    integer scores over a long context) and an above-bin list larger than its LDS
    capacity take the general multi-pass select; results must still be exact."""
    rng = np.random.default_rng(11)
    n = 12000
    krow = bf16_round(rng.standard_normal(128))
    k = [np.broadcast_to(krow, (1, n, 128)).copy()]
    v = [bf16_round(rng.standard_normal((1, n, 128)))]
    case = TinyCase(k, v, bf16_round(rng.standard_normal((1, 4, 128))))
    dev = DeviceCase.of_tiny(case)
    gidx = dev.index(np.array([700], np.int32), 700)
    assert np.array_equal(gidx[0], np.broadcast_to(np.arange(700), (4, 700)))
    case = random_case(rng, batch=2, hq=4, hkv=1, lens=[20000, 17000], integer=True, lo=-1, hi=1)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    run_and_check(dev, cache, case.q, np.array([2000, 400], np.int32), 2000, strict=True, check_dense=False,
                  tag="fallback")


@pytest.mark.parametrize("integer", [False, True], ids=["random", "integer-ties"])
def test_large_k_all_keys(integer):
    """k a large share of N (2x-3x sparsity): the score pass writes every key and the
    select radix-selects over the key rows; exact, ties included on integer inputs."""
    rng = np.random.default_rng(14)
    case = random_case(rng, batch=2, hq=8, hkv=2, lens=[5000, 3333], integer=integer, lo=-2, hi=2)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    run_and_check(dev, cache, case.q, np.array([2500, 1111], np.int32), 2500, strict=integer,
                  check_dense=False, tag="all-keys")


def test_select_sample_bound_too_high():
    """Every page the sampling pass looks at (one in four here) holds high scores and
    the other pages low ones, so the sample's lower bound is reached by fewer than k
    tokens of the row; the select must notice and still return the exact top k."""
    rng = np.random.default_rng(12)
    n, hq = 4096, 4
    q = bf16_round(rng.standard_normal((1, hq, 128)))
    u = q[0].sum(axis=0)
    u /= np.linalg.norm(u)
    page = np.arange(n) // 16
    high = (page % 4) == 0
    k = np.where(high[:, None], 8.0 * u[None, :] + 0.5 * rng.standard_normal((n, 128)),
                 0.1 * rng.standard_normal((n, 128)))
    case = TinyCase([bf16_round(k)[None]], [bf16_round(rng.standard_normal((1, n, 128)))], q,
                    layout="contiguous")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    gidx, _, _, _ = run_and_check(dev, cache, case.q, np.array([400], np.int32), 400, check_dense=False,
                                  tag="sample-bound")
    assert np.all(gidx[0] >= 0)


def test_select_block_bound_above_kth():
    """The first workgroup's sample pages hold the highest keys of the row and the rest
    of that workgroup low ones, so its bound lies above the k-th key while the other
    workgroups still deliver enough candidates; the select must detect the bound it
    cannot trust and still return the exact top k."""
    rng = np.random.default_rng(13)
    n, hq = 16384, 4
    q = bf16_round(rng.standard_normal((1, hq, 128)))
    u = q[0].sum(axis=0)
    u /= np.linalg.norm(u)
    t = np.arange(n)
    high = (t < 4096) & ((t % 512) < 128)                     # the first workgroup's sample pages
    low = (t < 4096) & ~high
    amp = np.where(high, 6.0, np.where(low, 0.0, 3.0))
    noise = np.where(low, 0.1, 0.3)[:, None] * rng.standard_normal((n, 128))
    k = amp[:, None] * u[None, :] + noise
    case = TinyCase([bf16_round(k)[None]], [bf16_round(rng.standard_normal((1, n, 128)))], q,
                    layout="shuffled")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    gidx, _, _, _ = run_and_check(dev, cache, case.q, np.array([1000], np.int32), 1000, check_dense=False,
                                  tag="block-bound")
    assert np.all(np.isin(np.nonzero(high)[0], gidx[0]))


def test_graph_replay_matches_eager():
    """A decode step (index -> attend) and dense decode captured in one HIP graph and
    replayed several times, with eager work and synchronisation between replays:
    every replay must reproduce the eager results bit for bit."""
    wl = synth.config(2, n=5000, batch=2)
    dev = DeviceCase.of_workload(wl)
    kps = i32_tensor(wl.k_per_seq())
    k_max = wl.k_max()
    B, hq = wl.batch, wl.num_q_heads
    idx = torch.empty((B, hq, k_max), dtype=torch.int32, device="cuda")
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    dn = torch.empty_like(out)
    ws_i = torch.empty(sdi.index_topk_workspace_bytes(dev.kv, hq, k_max), dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, sdi.attend_workspace_bytes(dev.kv, hq, k_max)), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(sdi.dense_workspace_bytes(dev.kv, hq), dtype=torch.uint8, device="cuda")

    def step():
        st = torch.cuda.current_stream()
        sdi.index_topk(dev.kv, dev.q, kps, k_max, idx_out=idx, workspace=ws_i, stream=st)
        sdi.attend(dev.kv, dev.q, idx, kps, out=out, workspace=ws_a, stream=st)
        sdi.dense(dev.kv, dev.q, out=dn, workspace=ws_d, stream=st)

    step()
    torch.cuda.synchronize()
    want = (idx.clone(), out.clone(), dn.clone())
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        idx.fill_(-7); out.fill_(float("nan")); dn.fill_(float("nan"))
        ws_i.fill_(0xAB)                                     # stale scratch must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph] replay {rep}")
        assert torch.equal(idx, want[0]) and torch.equal(out, want[1]) and torch.equal(dn, want[2]), rep
