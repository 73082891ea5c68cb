"""GPU parity for query-group sizes the five workloads do not use: G = 1 (one q head per
kv head), G = 7 (a partial head block), G = 16 and G = 32 (several head blocks per kv
head in the score pass, the dense kernel, the label indexer and the page bounds).
Exact indexer, attend and dense, the label indexer and the Quest page selection, each
against the oracle by the rules of the other parity tests."""
import numpy as np
import pytest

import oracle
from helpers import random_case

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase
    from test_gpu_labels import channels_by_magnitude, check_labels
    from test_gpu_parity import run_and_check
    from test_gpu_quest import check_quest

SHAPES = [(4, 4), (14, 2), (32, 2), (32, 1)]


@pytest.mark.parametrize("hq,hkv", SHAPES, ids=[f"Hq{a}-Hkv{b}" for a, b in SHAPES])
def test_group_sizes(hq, hkv):
    rng = np.random.default_rng(100 + hq * 8 + hkv)
    case = random_case(rng, batch=2, hq=hq, hkv=hkv, lens=[2500, 4100])
    dev = DeviceCase.of_tiny(case)
    cache = oracle.Cache(case.k_cache, case.v_cache, case.page_table, case.lens)
    kps = np.array([50, 82], np.int32)
    tag = f"G={hq // hkv}"
    run_and_check(dev, cache, case.q, kps, 82, tag=tag)
    channels = channels_by_magnitude(case.k_cache, case.page_table, case.lens, hkv)
    check_labels(dev, cache, case.q, channels, kps, 82, tag=f"{tag} labels")
    check_quest(dev, cache, case.q, np.array([4, 6], np.int32), 6, tag=f"{tag} quest")
