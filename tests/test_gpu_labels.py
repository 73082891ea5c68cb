"""GPU parity of the lightweight (reduced-channel label) indexer against the oracle.

Label rows are a gather of key channels, so they must equal the cache bits.  The
selection is the exact top-k of the reduced-channel scores s~ (oracle.label_scores,
then oracle.topk), compared with the token rule: identical except entries within
the tie window of the k-th s~; integer inputs are strict, ties included.  Attention
over the GPU's list is compared with the oracle's attention over the same list.
"""
import numpy as np
import pytest

import oracle
import synth
from helpers import bf16_round, random_case
from parity import check_close, check_indices

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi


def channels_by_magnitude(k_cache, page_table, seq_lens, hkv, r=16):
    """Per kv head the r channels of largest mean |K| over the cached rows, ascending
    (a plain offline calibration)."""
    ch = np.zeros((hkv, r), np.int32)
    vals = (k_cache.astype(np.uint32) << 16).view(np.float32)
    for g in range(hkv):
        acc = np.zeros(128)
        for b in range(len(seq_lens)):
            n = int(seq_lens[b])
            pages = page_table[b, :-(-n // 16)]
            rows = vals[pages, g].reshape(-1, 128)[:n]
            acc += np.abs(rows).sum(axis=0)
        ch[g] = np.sort(np.argsort(-acc, kind="stable")[:r])
    return ch


def check_labels(dev, cache, q, channels, k_per_seq, k_max, strict=False, tag=""):
    print(f"[case] {tag} B={cache.batch} N={list(cache.sl)[:6]} k={list(k_per_seq)[:6]} k_max={k_max}", flush=True)
    lab, gidx = dev.label_index(channels, k_per_seq, k_max)
    for b in range(cache.batch):
        for p in cache.pt[b, :-(-int(cache.sl[b]) // 16)]:
            for g in range(cache.num_kv_heads):
                assert np.array_equal(lab[p, g], cache.k[p, g][:, channels[g]]), f"{tag}: labels of page {p}"
    s = oracle.label_scores(cache, q, channels)
    oidx, kth = oracle.topk(np.nan_to_num(s, nan=-np.inf), cache.sl, k_per_seq, k_max)
    check_indices(gidx, oidx, s, kth, cache.sl, k_per_seq, strict=strict)
    out = dev.attend(gidx, k_per_seq)
    check_close(out, oracle.attend(cache, q, gidx), what=f"{tag} attend(label idx)")
    return gidx


@pytest.mark.parametrize("cfg,kw", [
    (3, dict(n=3001, batch=2)),
    (2, dict(n=4100, batch=2)),
    (5, dict(n=6000, batch=6, steps=1)),
], ids=["C3-small-outliers", "C2-small", "C5-small-ragged"])
def test_label_index_configs(cfg, kw):
    wl = synth.config(cfg, **kw)
    dev = DeviceCase.of_workload(wl)
    cache = oracle.Cache.of(wl)
    ch = channels_by_magnitude(wl.k_cache, wl.page_table, wl.seq_lens, wl.num_kv_heads)
    check_labels(dev, cache, wl.q, ch, wl.k_per_seq(), wl.k_max(), tag=f"C{cfg}-labels")


@pytest.mark.parametrize("kvec,k_max", [([40, 120, 2], 120), ([2000, 900, 5], 2000)],
                         ids=["candidates", "all-keys"])
def test_label_index_integer_strict(kvec, k_max):
    """Integer inputs: every s~ exact in fp32, many ties (lower index first).  Small k
    overflows the slot lists through the ties and re-scores from the label rows; large
    k takes the all-keys path."""
    rng = np.random.default_rng(51)
    case = random_case(rng, batch=3, hq=8, hkv=2, lens=[3000, 4100, 17], layout="fragmented",
                       integer=True, lo=-1, hi=1)
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    ch = np.stack([np.sort(rng.choice(128, 16, replace=False)) for _ in range(2)]).astype(np.int32)
    check_labels(dev, cache, case.q, ch, np.array(kvec, np.int32), k_max, strict=True, tag="labels-int")


def test_label_current_page_update():
    """After an appended token, rebuilding only the current pages equals a full build."""
    rng = np.random.default_rng(52)
    case = random_case(rng, batch=3, hq=4, hkv=2, lens=[40, 161, 95], layout="shuffled")
    dev = DeviceCase.of_tiny(case)
    ch = i32_tensor(np.stack([np.arange(16) * 8, np.arange(16) * 8 + 3]).astype(np.int32))
    n = case.lens.copy()
    stale = sdi.label_build(dev.kv, ch)
    pages = case.page_table[np.arange(3), n // 16]
    kr = bf16_round(rng.standard_normal((3, 2, 128)))
    from device import bf16_tensor
    from helpers import bf16_bits
    dev.k[torch.from_numpy(pages).cuda(), :, torch.from_numpy(n % 16).cuda(), :] = bf16_tensor(bf16_bits(kr))
    dev.sl += 1
    dev.kv.n_max = int(n.max()) + 1
    full = sdi.label_build(dev.kv, ch)
    sdi.label_build(dev.kv, ch, stale, current_pages_only=True)
    torch.cuda.synchronize()
    used = torch.from_numpy(np.concatenate([case.page_table[b, :-(-(int(n[b]) + 1) // 16)]
                                            for b in range(3)]).astype(np.int64)).cuda()
    assert torch.equal(stale.view(torch.int16)[used], full.view(torch.int16)[used])
