"""Full-size parity of the lightweight indexer, the Quest-style page selection and
the stochastic selection, each in the launch configuration the benchmark times:
every row runs on the GPU (with properties checked on all of them), and the oracle
checks every head of sampled sequences, by the rules of the smaller tests."""
import numpy as np
import pytest

import oracle
import synth
from parity import check_close, check_indices

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi
    from test_gpu_quest import compare_quest


def _say(*a):
    print(*a, flush=True)


def _sub_cache(wl, sub):
    return oracle.Cache(wl.k_cache, wl.v_cache, wl.page_table[sub], wl.seq_lens[sub], wl.num_kv_heads)


def _rows_ascending(idx, lens, counts):
    for b in range(idx.shape[0]):
        for h in range(idx.shape[1]):
            c = int(counts[b])
            row = idx[b, h]
            assert np.all(row[c:] == -1) and np.all(np.diff(row[:c]) > 0), (b, h)
            assert c == 0 or (row[0] >= 0 and row[c - 1] < lens[b]), (b, h)


def _calibrated_channels(wl, r=16, sample=2048):
    """Per kv head the r channels of largest mean |K| over the first tokens of sequence 0."""
    n = min(sample, int(wl.seq_lens[0]))
    pages = wl.page_table[0, :-(-n // 16)]
    vals = (wl.k_cache[pages].astype(np.uint32) << 16).view(np.float32)
    return np.stack([np.sort(np.argsort(-np.abs(vals[:, g].reshape(-1, 128)[:n]).mean(axis=0), kind="stable")[:r])
                     for g in range(wl.num_kv_heads)]).astype(np.int32)


def test_labels_full_size():
    wl = synth.config(2)
    dev = DeviceCase.of_workload(wl)
    kps, k_max = wl.k_per_seq(), wl.k_max()
    ch = _calibrated_channels(wl)
    _say("[case] C2 full size: label build + label index + attend on the GPU")
    lab, gidx = dev.label_index(ch, kps, k_max)
    out = dev.attend(gidx, kps)
    _rows_ascending(gidx, wl.seq_lens, np.minimum(kps, wl.seq_lens))
    sub = np.array([1, 6])
    for b in sub:
        pages = wl.page_table[b, :-(-int(wl.seq_lens[b]) // 16)]
        for g in range(wl.num_kv_heads):
            assert np.array_equal(lab[pages, g], wl.k_cache[pages, g][:, :, ch[g]]), (b, g)
    cache, q = _sub_cache(wl, sub), wl.q[sub]
    s = oracle.label_scores(cache, q, ch)
    oidx, kth = oracle.topk(s, cache.sl, kps[sub], k_max)
    check_indices(gidx[sub], oidx, s, kth, cache.sl, kps[sub])
    check_close(out[sub], oracle.attend(cache, q, gidx[sub]), what="C2 attend(label idx)")


def test_quest_full_size():
    wl = synth.config(2)
    dev = DeviceCase.of_workload(wl)
    m = -(-int(wl.k_max()) // 16)
    mps = np.full(wl.batch, m, np.int32)
    _say(f"[case] C2 full size: Quest summaries + page selection (m = {m}) + attend on the GPU")
    _, summ_bits, gtok = dev.quest(mps, m)
    out = dev.attend(gtok)
    for b in range(wl.batch):                                 # m whole pages, the current one among them
        P = -(-int(wl.seq_lens[b]) // 16)
        for h in range(wl.num_q_heads):
            pages = np.unique(gtok[b, h][gtok[b, h] >= 0] // 16)
            assert len(pages) == m and pages[-1] == P - 1, (b, h)
    sub = np.array([2, 7])
    cache, q = _sub_cache(wl, sub), wl.q[sub]
    compare_quest(summ_bits, gtok[sub], cache, q, mps[sub], m, tag="C2-full-quest")
    check_close(out[sub], oracle.attend(cache, q, gtok[sub]), what="C2 attend(quest tokens)")


@pytest.mark.parametrize("cfg,sample", [(2, [0, 3]), (5, [4, 17])], ids=["C2-full", "C5-full"])
def test_sampled_full_size(cfg, sample):
    wl = synth.config(cfg)
    dev = DeviceCase.of_workload(wl)
    k = wl.k_per_seq()
    kd, sv = (k + 1) // 2, k // 2
    kd_max, s_max = int(kd.max()), max(1, int(sv.max()))
    rng = np.random.default_rng(66 + cfg)
    draws = rng.integers(0, 2 ** 32, size=(wl.batch, wl.num_q_heads, s_max), dtype=np.uint64).astype(np.uint32)
    _say(f"[case] C{cfg} full size: top-{kd_max} + {s_max} draws + two-list attend on the GPU")
    idx = dev.index(kd, kd_max)
    d_idx, d_kd, d_sv = i32_tensor(idx), i32_tensor(kd), i32_tensor(sv)
    gs, gw = sdi.sample_residual(dev.kv, d_idx, d_kd, torch.from_numpy(draws.view(np.int32)).cuda(), d_sv)
    out = sdi.attend_sampled(dev.kv, dev.q, d_idx, d_kd, gs, gw, d_sv)
    torch.cuda.synchronize()
    gs, gw, out = gs.cpu().numpy(), gw.cpu().numpy(), out.cpu().numpy()
    lens = wl.seq_lens
    for b in range(wl.batch):                                 # every drawn token is outside its row's kept set
        for h in range(wl.num_q_heads):
            kept = idx[b, h][idx[b, h] >= 0]
            drawn = gs[b, h, :sv[b]]
            assert np.all(drawn >= 0) and np.all(drawn < lens[b]) and not np.isin(drawn, kept).any(), (b, h)
            assert np.all(gs[b, h, sv[b]:] == -1)
    sub = np.array(sample)
    os_, ow = oracle.sample_residual(idx[sub], kd[sub], lens[sub], draws[sub], sv[sub])
    assert np.array_equal(gs[sub], os_)
    assert np.all(np.abs(gw[sub] - ow) <= 2.0 ** -23 * ow)
    cache, q = _sub_cache(wl, sub), wl.q[sub]
    check_close(out[sub], oracle.attend_sampled(cache, q, idx[sub], gs[sub], ow), what=f"C{cfg} attend_sampled")


def test_next_rows_graph_replay_matches_eager():
    """The label step (current-page label update, label index, attend), the Quest step
    (current-page summaries, page selection, attend) and the stochastic step (index,
    draws, two-list attend) captured in one HIP graph and replayed several times, with
    eager work and synchronisation between replays: every replay reproduces the eager
    results bit for bit."""
    wl = synth.config(2, n=5000, batch=2)
    dev = DeviceCase.of_workload(wl)
    B, hq = wl.batch, wl.num_q_heads
    k = wl.k_per_seq()
    k_max = int(k.max())
    kps = i32_tensor(k)
    ch = i32_tensor(_calibrated_channels(wl))
    labels = sdi.label_build(dev.kv, ch)
    summary = sdi.quest_summarize(dev.kv)
    m = -(-k_max // 16)
    mps, tps = i32_tensor(np.full(B, m, np.int32)), i32_tensor(np.full(B, 16 * m, np.int32))
    kd, sv = i32_tensor((k + 1) // 2), i32_tensor(k // 2)
    kd_max, s_max = (k_max + 1) // 2, max(1, k_max // 2)
    rng = np.random.default_rng(67)
    draws = torch.from_numpy(rng.integers(0, 2 ** 32, size=(B, hq, s_max), dtype=np.uint64)
                             .astype(np.uint32).view(np.int32)).cuda()
    cuda = dict(device="cuda")
    lidx = torch.empty((B, hq, k_max), dtype=torch.int32, **cuda)
    qidx = torch.empty((B, hq, 16 * m), dtype=torch.int32, **cuda)
    kidx = torch.empty((B, hq, kd_max), dtype=torch.int32, **cuda)
    smp = torch.empty((B, hq, s_max), dtype=torch.int32, **cuda)
    wt = torch.empty((B, hq), dtype=torch.float32, **cuda)
    outs = [torch.empty((B, hq, 128), dtype=torch.float32, **cuda) for _ in range(3)]
    ws_i = torch.empty(sdi.index_topk_workspace_bytes(dev.kv, hq, k_max), dtype=torch.uint8, **cuda)
    ws_a = torch.empty(max(1, sdi.attend_workspace_bytes(dev.kv, hq, 16 * m)), dtype=torch.uint8, **cuda)
    ws_q = torch.empty(max(1, sdi.load_library().sparse_decode_quest_select_workspace(
        __import__("ctypes").byref(dev.kv.struct()), hq, m)), dtype=torch.uint8, **cuda)
    ws_s = torch.empty(max(1, sdi.attend_sampled_workspace_bytes(dev.kv, hq, kd_max, s_max)), dtype=torch.uint8,
                       **cuda)

    def step():
        st = torch.cuda.current_stream()
        sdi.label_build(dev.kv, ch, labels, current_pages_only=True, stream=st)
        sdi.label_index_topk(dev.kv, dev.q, labels, ch, kps, k_max, idx_out=lidx, workspace=ws_i, stream=st)
        sdi.attend(dev.kv, dev.q, lidx, kps, out=outs[0], workspace=ws_a, stream=st)
        sdi.quest_summarize(dev.kv, summary, current_pages_only=True, stream=st)
        sdi.quest_select(dev.kv, dev.q, summary, mps, m, idx_out=qidx, workspace=ws_q, stream=st)
        sdi.attend(dev.kv, dev.q, qidx, tps, out=outs[1], workspace=ws_a, stream=st)
        sdi.index_topk(dev.kv, dev.q, kd, kd_max, idx_out=kidx, workspace=ws_i, stream=st)
        sdi.sample_residual(dev.kv, kidx, kd, draws, sv, sample_out=smp, weight_out=wt, stream=st)
        sdi.attend_sampled(dev.kv, dev.q, kidx, kd, smp, wt, sv, out=outs[2], workspace=ws_s, stream=st)

    results = lambda: [t.clone() for t in (lidx, qidx, kidx, smp, wt, *outs)]
    step()
    torch.cuda.synchronize()
    want = results()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        for t in (lidx, qidx, kidx, smp):
            t.fill_(-7)
        for t in (wt, *outs):
            t.fill_(float("nan"))
        for t in (ws_i, ws_a, ws_q, ws_s):
            t.fill_(0xAB)                                    # stale scratch must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph] replay {rep}")
        got = results()
        for j, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), (rep, j)
