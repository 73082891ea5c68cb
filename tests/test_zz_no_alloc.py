"""The allocation-free attend entry point (sparse_decode_attend_noalloc) through the C
ABI against the workspace form (sparse_decode_attend) on the same inputs: two calls in
a row, the second with a smaller batch and fewer heads, both with rows long enough to
be split (so the fixed scratch holds their partials), and a short-row call that needs
no scratch.  Results must agree to the output tolerance (they come from the same
kernels, so they agree bit for bit).  A call beyond the scratch is refused before
anything is launched."""
import numpy as np
import pytest

from helpers import random_case
from parity import check_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from device import DeviceCase, i32_tensor
    import sparse_attention_decode_index_amd as sdi


def _rows(rng, lens, hq, k_max):
    return np.stack([np.stack([np.sort(rng.choice(n, size=min(k_max, n), replace=False)) for _ in range(hq)])
                     for n in lens]).astype(np.int32)


@pytest.mark.parametrize("shapes", [
    [(4, 16, 4, [20000, 9000, 15000, 3000], 3000), (2, 8, 2, [12000, 2500], 1500)],
    [(2, 8, 2, [5000, 800], 700), (3, 12, 3, [9000, 7000, 4000], 2100)],
], ids=["large-then-small", "short-rows-then-split"])
def test_noalloc_matches_workspace_form(shapes):
    rng = np.random.default_rng(31)
    for call, (B, hq, hkv, lens, k_max) in enumerate(shapes):
        print(f"[case] call {call}: B={B} Hq={hq} Hkv={hkv} N={lens} k_max={k_max}", flush=True)
        case = random_case(rng, batch=B, hq=hq, hkv=hkv, lens=lens, layout="fragmented")
        dev = DeviceCase.of_tiny(case)
        idx = _rows(rng, lens, hq, k_max)
        idx[0, 0, 5:9] = -1                                # holes are skipped in both forms
        kps = np.array([min(k_max, n) - 3 * b for b, n in enumerate(lens)], np.int32)
        idx_t, kps_t = i32_tensor(idx), i32_tensor(kps)
        want = sdi.attend(dev.kv, dev.q, idx_t, kps_t)
        got = sdi.attend_noalloc(dev.kv, dev.q, idx_t, kps_t)
        torch.cuda.synchronize()
        check_close(got.cpu().numpy(), want.cpu().numpy(), what=f"no-alloc call {call}")
        assert torch.equal(got, want), f"call {call}: not bit-identical to the workspace form"


def test_noalloc_rejects_calls_beyond_its_scratch():
    rng = np.random.default_rng(32)
    case = random_case(rng, batch=1, hq=4, hkv=1, lens=[300])
    dev = DeviceCase.of_tiny(case)
    # 16384 rows of 16 chunks each: 136 MB of partials, beyond the 32 MiB scratch
    q = torch.zeros((1, 16384, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.full((1, 16384, 4000), -1, dtype=torch.int32, device="cuda")
    with pytest.raises(sdi.SparseDecodeError) as e:
        sdi.attend_noalloc(dev.kv, q, idx)
    assert e.value.code == sdi.SDI_ERR_TOO_LARGE
    # the refused call launched nothing: a valid call still works after it
    idx = torch.from_numpy(np.arange(300, dtype=np.int32)[None, None].repeat(4, 1)).cuda()
    out = sdi.attend_noalloc(dev.kv, dev.q, idx)
    check_close(out.cpu().numpy(), sdi.attend(dev.kv, dev.q, idx).cpu().numpy(), what="after refusal")
