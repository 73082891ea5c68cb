"""GPU parity of stochastic index selection against the fp64 oracle.

The sampler maps each 32-bit draw to a token of the residual of a top-k row (the
tokens the row left out), so given the same row and the same draws the drawn
tokens must match the oracle's bit for bit, and the weight M / s' to within one
fp32 rounding.  The two-list attend (top-k entries weight 1, drawn entries weight
M / s') is compared with the oracle's estimate over the same lists.  Rows come
from the GPU's own top-k (already checked against the oracle elsewhere), so no
tie window enters.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import random_case
from parity import check_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi


def u32_draws(rng, shape):
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)


def check_sampled(dev, cache, q, idx, k_per_seq, draws, s_per_seq, tag=""):
    """Sampler and two-list attend against the oracle on the same top-k rows and draws."""
    print(f"[case] {tag} B={cache.batch} N={list(cache.sl)[:6]} k_max={idx.shape[2]} s_max={draws.shape[2]}",
          flush=True)
    d_idx, d_kps = i32_tensor(idx), i32_tensor(k_per_seq)
    d_draws = torch.from_numpy(draws.view(np.int32)).cuda()
    d_sps = i32_tensor(s_per_seq)
    gs, gw = sdi.sample_residual(dev.kv, d_idx, d_kps, d_draws, d_sps)
    out = sdi.attend_sampled(dev.kv, dev.q, d_idx, d_kps, gs, gw, d_sps)
    full = sdi.attend_sampled(dev.kv, dev.q, d_idx, d_kps, gs, gw)     # s_per_seq NULL: every draw entry read
    torch.cuda.synchronize()
    gs, gw, out, full = gs.cpu().numpy(), gw.cpu().numpy(), out.cpu().numpy(), full.cpu().numpy()
    os_, ow = oracle.sample_residual(idx, k_per_seq, cache.sl, draws, s_per_seq)
    assert np.array_equal(gs, os_), f"{tag}: drawn tokens differ"
    assert np.all(np.abs(gw - ow) <= 2.0 ** -23 * ow), f"{tag}: weights differ"
    want = oracle.attend_sampled(cache, q, idx, gs, ow)
    check_close(out, want, what=f"{tag} attend_sampled")
    check_close(full, want, what=f"{tag} attend_sampled (s_per_seq NULL)")
    return gs, gw, out


@pytest.mark.parametrize("cfg,kw", [
    (2, dict(n=4100, batch=2)),
    (5, dict(n=6000, batch=6, steps=1)),
    (3, dict(n=3001, batch=2)),
], ids=["C2-small", "C5-small-ragged", "C3-small"])
def test_sampled_configs(cfg, kw):
    """Half of each budget to the exact top-k, half to draws from the rest."""
    wl = synth.config(cfg, **kw)
    dev = DeviceCase.of_workload(wl)
    cache = oracle.Cache.of(wl)
    k = wl.k_per_seq()
    kdet = (k + 1) // 2
    k_max = int(kdet.max())
    idx = dev.index(kdet, k_max)
    svec = (k - kdet).astype(np.int32)
    rng = np.random.default_rng(61 + cfg)
    check_sampled(dev, cache, wl.q, idx, kdet, u32_draws(rng, (wl.batch, wl.q.shape[1], max(int(svec.max()), 1))),
                  svec, tag=f"C{cfg}-sampled")


def test_sampled_enumeration_is_dense():
    """Draws that hit every residual token once: weight 1, and the estimate is dense attention."""
    rng = np.random.default_rng(62)
    case = random_case(rng, batch=3, hq=8, hkv=2, lens=[300, 1000, 77], layout="fragmented")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    kvec = np.array([20, 64, 5], np.int32)
    idx = dev.index(kvec, 64)
    M = case.lens - kvec
    s_max = int(M.max())
    draws = np.zeros((3, 8, s_max), np.uint32)
    for b in range(3):
        draws[b, :, :M[b]] = [(r * 2 ** 32 + int(M[b]) - 1) // int(M[b]) for r in range(int(M[b]))]
    gs, gw, out = check_sampled(dev, cache, case.q, idx, kvec, draws, M.astype(np.int32), tag="enumerate")
    assert np.all(gw == 1.0)
    check_close(out, oracle.dense(cache, case.q), what="enumerated estimate vs dense")


def test_sampled_edges():
    """Empty residuals (k >= N), no draws, more draws asked than s_max, one-token sequences,
    and rows longer than 1024 entries (chunked attend)."""
    rng = np.random.default_rng(63)
    case = random_case(rng, batch=5, hq=4, hkv=1, lens=[1, 40, 700, 2000, 16], layout="shuffled")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    kvec = np.array([3, 40, 650, 900, 2], np.int32)
    idx = dev.index(kvec, 900)
    svec = np.array([5, 9, 0, 5000, 14], np.int32)
    _, gw, out = check_sampled(dev, cache, case.q, idx, kvec, u32_draws(rng, (5, 4, 300)), svec, tag="edges")
    assert np.all(gw[:2] == 0.0) and np.all(gw[2] == 0.0)           # empty residual; s = 0
    assert np.allclose(gw[3], (2000 - 900) / 300)                     # s clipped to s_max
    assert np.allclose(gw[4], 14 / 14)


def test_sampled_long_rows_searched_in_place():
    """A kept row longer than the LDS staging limit: the bisection reads the row in place."""
    rng = np.random.default_rng(64)
    case = random_case(rng, batch=1, hq=2, hkv=1, lens=[20000], layout="fragmented")
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    kvec = np.array([16000], np.int32)
    idx = dev.index(kvec, 16000)
    check_sampled(dev, cache, case.q, idx, kvec, u32_draws(rng, (1, 2, 500)), np.array([500], np.int32),
                  tag="long-row")


def test_sampled_argument_errors():
    rng = np.random.default_rng(65)
    case = random_case(rng, batch=1, hq=4, hkv=1, lens=[20])
    dev = DeviceCase.of_tiny(case)
    idx = i32_tensor(np.zeros((1, 4, 3), np.int32))
    with pytest.raises(ValueError):
        sdi.sample_residual(dev.kv, idx, i32_tensor([1]), torch.zeros((1, 4, 2), dtype=torch.int64, device="cuda"),
                            i32_tensor([1]))
