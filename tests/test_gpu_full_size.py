"""GPU parity at full size: every sequence, every query head and every decode step of
the workloads, in the launch configuration the benchmark times, against the fp64
oracle (comparison rules in tests/parity.py).

* Llama-3-8B-shaped layer (B8, 32/8 heads, N 32768, k 655) and long retrieval (B4,
  40/8 heads, N 131072, k 2621): one step, all rows.
* Extreme-sparsity sweep (B16, 32/8 heads, N 131072 growing 8 steps): every step at
  k = N/500, N/100, N/50 and N/20, plus dense decode (the k = N row); at the first
  step also the sparse path at k = N against dense decode.
* Agentic ragged batch (B32, 64/8 heads, N_i in [8192, 163840] growing 32 steps,
  k = ceil(N_i/50), fragmented pages): all 32 steps, in four tests of eight steps that
  share one cache (the tests run in file order; a later one advances the cache itself
  if run alone).

At each step the GPU's index rows are validated against the oracle's exact top-k,
the attend runs on the GPU's own list and on the oracle's list (each compared with
the oracle's attention over the same list), and dense decode is compared with the
oracle's dense attention.  k_max is the benchmark's: the largest k over all steps.
"""
import time

import numpy as np
import pytest

import oracle
import synth
from parity import check_close, check_indices

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase


def _say(*a):
    print(*a, flush=True)


def check_step(dev, wl, legs, tag, dense=True):
    """legs: (name, k rule, k_max) per sparsity level.  Returns the GPU dense output."""
    t0 = time.perf_counter()
    cache = oracle.Cache.of(wl)
    s = oracle.scores(cache, wl.q)
    swaps = []
    for name, rule, k_max in legs:
        kps = rule(wl.seq_lens)
        gidx = dev.index(kps, k_max)
        oidx, kth = oracle.topk(s, cache.sl, kps, k_max)
        swaps.append(check_indices(gidx, oidx, s, kth, cache.sl, kps))
        check_close(dev.attend(gidx, kps), oracle.attend(cache, wl.q, gidx), what=f"{tag} {name} attend(gpu idx)")
        check_close(dev.attend(oidx, kps), oracle.attend(cache, wl.q, oidx), what=f"{tag} {name} attend(oracle idx)")
    dn = None
    if dense:
        dn = dev.dense()
        check_close(dn, oracle.dense(cache, wl.q), what=f"{tag} dense")
    _say(f"[step] {tag} N={int(wl.seq_lens.min())}..{int(wl.seq_lens.max())} "
         f"legs={[l[0] for l in legs]} window swaps={swaps} ({time.perf_counter() - t0:.1f} s)")
    return dn


def test_llama_layer_every_row():
    wl = synth.config(2)
    _say("[case] Llama-3-8B layer, full size, every sequence")
    dev = DeviceCase.of_workload(wl)
    kps = wl.k_per_seq()
    check_step(dev, wl, [("N/50", synth.k_half_up(50), wl.k_max())], "C2")
    gidx = dev.index(kps, wl.k_max())
    for b in range(wl.batch):                  # the planted keys are in every head's selection
        for h in range(wl.num_q_heads):
            assert set(wl.meta["planted_positions"][(b, h // wl.group)]) <= set(gidx[b, h].tolist())


def test_long_retrieval_every_row():
    wl = synth.config(3)
    _say("[case] long retrieval, full size, every sequence")
    dev = DeviceCase.of_workload(wl)
    check_step(dev, wl, [("N/50", synth.k_half_up(50), wl.k_max())], "C3")


class GrowingRun:
    """A growing workload's cache, on the host (oracle) and on the device, shared by the
    tests that check consecutive ranges of its steps."""
    runs = {}

    @classmethod
    def at(cls, cfg, step):
        run = cls.runs.get(cfg)
        if run is None or run[0].step > step:
            cls.runs.pop(cfg, None)
            torch.cuda.empty_cache()
            wl = synth.config(cfg)
            run = cls.runs[cfg] = (wl, DeviceCase.of_workload(wl))
        wl, dev = run
        while wl.step < step:
            rows = wl.advance()
            dev.append(rows, wl.q, wl.n_max)
        return wl, dev

    @classmethod
    def drop(cls, cfg):
        cls.runs.pop(cfg, None)
        torch.cuda.empty_cache()


def k_legs(wl, rules):
    """(name, rule, k_max) with the benchmark's k_max: the largest k over all steps."""
    last = wl.seq_lens - wl.step + (wl.steps - 1)
    return [(name, rule, int(rule(last).max())) for name, rule in rules]


SWEEP_RULES = [(f"N/{r}", synth.k_half_up(r)) for r in (500, 100, 50, 20)]


@pytest.mark.parametrize("first", [0, 4], ids=["steps0-3", "steps4-7"])
def test_sweep_every_step_every_k(first):
    _say(f"[case] sparsity sweep, full size, steps {first}..{first + 3}, k = N/500, N/100, N/50, N/20 and dense")
    for step in range(first, first + 4):
        wl, dev = GrowingRun.at(4, step)
        dn = check_step(dev, wl, k_legs(wl, SWEEP_RULES), f"C4 step {step}")
        if step == 0:                          # k = N: the sparse path reproduces dense decode
            kps = wl.seq_lens.copy()
            gidx = dev.index(kps, wl.n_max)
            assert all(np.array_equal(gidx[b, h], np.arange(wl.n_max)) for b in range(wl.batch)
                       for h in range(wl.num_q_heads))
            check_close(dev.attend(gidx, kps), dn, what="C4 k=N sparse vs dense")
    if first == 4:
        GrowingRun.drop(4)


@pytest.mark.parametrize("first", [0, 8, 16, 24], ids=["steps0-7", "steps8-15", "steps16-23", "steps24-31"])
def test_agentic_every_step(first):
    _say(f"[case] agentic ragged batch, full size, steps {first}..{first + 7}, every sequence")
    for step in range(first, first + 8):
        wl, dev = GrowingRun.at(5, step)
        check_step(dev, wl, k_legs(wl, [("ceil(N/50)", synth.k_ceil(50))]), f"C5 step {step}")
    if first == 24:
        GrowingRun.drop(5)
