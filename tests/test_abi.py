"""The C ABI on the host: the library loads, exports every declared symbol, and every
argument error is reported before anything is launched (no GPU needed: the
checks return before any HIP call, and the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import sparse_attention_decode_index_amd as sdi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sparse_decode.h")
FAKE = 0x10000                                 # a non-NULL address that is never touched


@pytest.fixture(scope="module")
def lib():
    return sdi.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^SDI_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)))


def kv(**over):
    base = dict(k_cache=FAKE, v_cache=FAKE, page_table=FAKE, seq_lens=FAKE, batch=2, num_kv_heads=2,
                head_dim=128, page_size=16, max_pages_per_seq=10, num_pages=40, n_max=150)
    base.update(over)
    return sdi.SdiKV(**base)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(sdi.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header():
    # 4 pointers + 7 int32, naturally aligned
    assert ctypes.sizeof(sdi.SdiKV) == 4 * 8 + 7 * 4 + 4


def test_strerror_covers_every_code(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = sdi.strerror(code)
        assert s and "unknown" not in s
    assert "unknown" in sdi.strerror(42)


def test_workspace_sizes(lib):
    k = kv()
    n1 = lib.sparse_decode_index_topk_workspace(ctypes.byref(k), 8, 5)
    # per row: a 32-bit key row (padded to 128 tokens), then per 512-token slot a 1280-byte
    # record: 192 32-bit keys, a count, the slot's lower bound, its largest key, a pad word
    # and 192 16-bit positions, padded to whole 128-byte lines
    assert n1 == 2 * 8 * (256 * 4 + 1 * 1280)
    assert lib.sparse_decode_attend_workspace(ctypes.byref(k), 8, 1024) == 0         # one chunk: no partials
    assert lib.sparse_decode_attend_workspace(ctypes.byref(k), 8, 1025) == 2 * 8 * 5 * 130 * 4   # 256-entry chunks
    assert lib.dense_decode_workspace(ctypes.byref(k), 8) == 2 * 8 * 1 * 130 * 4      # one 4096-token chunk
    assert lib.sparse_decode_attend_workspace(None, 8, 5) == 0


def call_index(lib, k, hq=8, k_max=5, q=FAKE, kps=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40):
    return lib.sparse_decode_index_topk(ctypes.byref(k) if k is not None else None, q, hq, kps, k_max, out, ws,
                                        nbytes, None)


def call_attend(lib, k, hq=8, k_max=5, q=FAKE, idx=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40):
    return lib.sparse_decode_attend(ctypes.byref(k) if k is not None else None, q, hq, idx, None, k_max, 0.1, out,
                                    ws, nbytes, None)


def call_dense(lib, k, hq=8, q=FAKE, out=FAKE, ws=FAKE, nbytes=1 << 40):
    return lib.dense_decode(ctypes.byref(k) if k is not None else None, q, hq, 0.1, out, ws, nbytes, None)


@pytest.mark.parametrize("over,code", [
    (dict(head_dim=64), sdi.SDI_ERR_SHAPE),
    (dict(page_size=32), sdi.SDI_ERR_SHAPE),
    (dict(batch=0), sdi.SDI_ERR_SHAPE),
    (dict(num_kv_heads=0), sdi.SDI_ERR_SHAPE),
    (dict(n_max=0), sdi.SDI_ERR_SHAPE),
    (dict(num_pages=0), sdi.SDI_ERR_SHAPE),
    (dict(max_pages_per_seq=9), sdi.SDI_ERR_SHAPE),       # 150 tokens need 10 pages
    (dict(num_pages=1 << 30), sdi.SDI_ERR_SHAPE),         # row numbers would overflow 32 bits
    (dict(k_cache=None), sdi.SDI_ERR_NULL),
    (dict(page_table=None), sdi.SDI_ERR_NULL),
    (dict(seq_lens=None), sdi.SDI_ERR_NULL),
])
def test_cache_errors(lib, over, code):
    k = kv(**over)
    assert call_index(lib, k) == code
    assert call_attend(lib, k) == code
    assert call_dense(lib, k) == code


def test_index_does_not_need_values(lib):
    # v_cache NULL is an error for attend/dense only; index still stops at its next check
    k = kv(v_cache=None)
    assert call_attend(lib, k) == sdi.SDI_ERR_NULL
    assert call_dense(lib, k) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, k_max=0) == sdi.SDI_ERR_K


def test_argument_errors(lib):
    k = kv()
    assert call_index(lib, None) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, q=None) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, kps=None) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, out=None) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, ws=None) == sdi.SDI_ERR_NULL
    assert call_index(lib, k, hq=7) == sdi.SDI_ERR_SHAPE      # not a multiple of 2 kv heads
    assert call_index(lib, k, hq=0) == sdi.SDI_ERR_SHAPE
    assert call_index(lib, k, k_max=0) == sdi.SDI_ERR_K
    need = lib.sparse_decode_index_topk_workspace(ctypes.byref(k), 8, 5)
    assert call_index(lib, k, nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE
    assert call_attend(lib, k, idx=None) == sdi.SDI_ERR_NULL
    assert call_attend(lib, k, out=None) == sdi.SDI_ERR_NULL
    assert call_attend(lib, k, k_max=0) == sdi.SDI_ERR_K
    assert call_attend(lib, k, hq=3) == sdi.SDI_ERR_SHAPE
    need = lib.sparse_decode_attend_workspace(ctypes.byref(k), 8, 2000)
    assert need > 0 and call_attend(lib, k, k_max=2000, nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE
    assert call_attend(lib, k, k_max=2000, ws=None) == sdi.SDI_ERR_NULL
    assert call_dense(lib, k, out=None) == sdi.SDI_ERR_NULL
    need = lib.dense_decode_workspace(ctypes.byref(k), 8)
    assert call_dense(lib, k, nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE


def test_quest_sizes_and_errors(lib):
    k = kv()
    # summaries: min and max row (2 x 128 bf16) per (physical page, kv head)
    assert lib.sparse_decode_quest_summary_bytes(ctypes.byref(k)) == 40 * 2 * 2 * 128 * 2
    # select workspace per (b, q head): one key per page (page rows padded to 64), then the page list
    assert lib.sparse_decode_quest_select_workspace(ctypes.byref(k), 8, 6) == 2 * 8 * (64 * 4 + 6 * 4)
    assert lib.sparse_decode_quest_select_workspace(ctypes.byref(k), 8, 0) == 0
    assert lib.sparse_decode_quest_summarize(None, FAKE, 0, None) == sdi.SDI_ERR_NULL
    assert lib.sparse_decode_quest_summarize(ctypes.byref(k), None, 0, None) == sdi.SDI_ERR_NULL
    assert lib.sparse_decode_quest_summarize(ctypes.byref(kv(head_dim=64)), FAKE, 0, None) == sdi.SDI_ERR_SHAPE

    def sel(hq=8, q=FAKE, summ=FAKE, pps=FAKE, pmax=6, out=FAKE, ws=FAKE, nbytes=1 << 40):
        return lib.sparse_decode_quest_select(ctypes.byref(k), q, hq, summ, pps, pmax, out, ws, nbytes, None)
    assert sel(q=None) == sdi.SDI_ERR_NULL
    assert sel(summ=None) == sdi.SDI_ERR_NULL
    assert sel(pps=None) == sdi.SDI_ERR_NULL
    assert sel(out=None) == sdi.SDI_ERR_NULL
    assert sel(ws=None) == sdi.SDI_ERR_NULL
    assert sel(hq=3) == sdi.SDI_ERR_SHAPE
    assert sel(pmax=0) == sdi.SDI_ERR_K
    need = lib.sparse_decode_quest_select_workspace(ctypes.byref(k), 8, 6)
    assert sel(nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE


def test_label_sizes_and_errors(lib):
    k = kv()
    assert lib.sparse_decode_label_bytes(ctypes.byref(k)) == 40 * 2 * 16 * 16 * 2   # 16 rows x 16 channels
    assert lib.sparse_decode_label_build(ctypes.byref(k), None, FAKE, 0, None) == sdi.SDI_ERR_NULL
    assert lib.sparse_decode_label_build(ctypes.byref(k), FAKE, None, 0, None) == sdi.SDI_ERR_NULL
    assert lib.sparse_decode_label_build(ctypes.byref(kv(page_size=8)), FAKE, FAKE, 0, None) == sdi.SDI_ERR_SHAPE

    def idx(hq=8, q=FAKE, lab=FAKE, ch=FAKE, kps=FAKE, k_max=5, out=FAKE, ws=FAKE, nbytes=1 << 40):
        return lib.sparse_decode_label_index_topk(ctypes.byref(k), q, hq, lab, ch, kps, k_max, out, ws, nbytes, None)
    for over in (dict(q=None), dict(lab=None), dict(ch=None), dict(kps=None), dict(out=None), dict(ws=None)):
        assert idx(**over) == sdi.SDI_ERR_NULL
    assert idx(hq=5) == sdi.SDI_ERR_SHAPE
    assert idx(k_max=0) == sdi.SDI_ERR_K
    need = lib.sparse_decode_index_topk_workspace(ctypes.byref(k), 8, 5)
    assert idx(nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE


def test_sample_sizes_and_errors(lib):
    k = kv()
    # two-list rows of k_max + s_max entries: one workgroup up to 1024, 256-entry chunks beyond
    assert lib.sparse_decode_attend_sampled_workspace(ctypes.byref(k), 8, 600, 424) == 0
    assert lib.sparse_decode_attend_sampled_workspace(ctypes.byref(k), 8, 600, 425) == 2 * 8 * 5 * 130 * 4
    assert lib.sparse_decode_attend_sampled_workspace(ctypes.byref(k), 8, 600, 0) == 0

    def smp(hq=8, idx=FAKE, kps=FAKE, k_max=5, draws=FAKE, sps=FAKE, s_max=7, out=FAKE, w=FAKE, kvv=k):
        return lib.sparse_decode_sample_residual(ctypes.byref(kvv), hq, idx, kps, k_max, draws, sps, s_max, out, w,
                                                 None)
    for over in (dict(idx=None), dict(kps=None), dict(draws=None), dict(sps=None), dict(out=None), dict(w=None)):
        assert smp(**over) == sdi.SDI_ERR_NULL
    assert smp(hq=3) == sdi.SDI_ERR_SHAPE
    assert smp(kvv=kv(head_dim=64)) == sdi.SDI_ERR_SHAPE
    assert smp(k_max=0) == sdi.SDI_ERR_K
    assert smp(s_max=0) == sdi.SDI_ERR_K

    def att(hq=8, q=FAKE, idx=FAKE, kps=FAKE, k_max=600, sm=FAKE, w=FAKE, s_max=500, out=FAKE, ws=FAKE,
            nbytes=1 << 40):
        return lib.sparse_decode_attend_sampled(ctypes.byref(k), q, hq, idx, kps, k_max, sm, w, FAKE, s_max,
                                                ctypes.c_float(0.1), out, ws, nbytes, None)
    for over in (dict(q=None), dict(idx=None), dict(sm=None), dict(w=None), dict(out=None), dict(ws=None)):
        assert att(**over) == sdi.SDI_ERR_NULL
    assert att(hq=5) == sdi.SDI_ERR_SHAPE
    assert att(s_max=0) == sdi.SDI_ERR_K
    assert att(k_max=0) == sdi.SDI_ERR_K
    need = lib.sparse_decode_attend_sampled_workspace(ctypes.byref(k), 8, 600, 500)
    assert att(nbytes=need - 1) == sdi.SDI_ERR_WORKSPACE
    assert lib.sparse_decode_attend_sampled(ctypes.byref(kv(v_cache=None)), FAKE, 8, FAKE, FAKE, 600, FAKE, FAKE,
                                            FAKE, 500, ctypes.c_float(0.1), FAKE, FAKE, 1 << 40,
                                            None) == sdi.SDI_ERR_NULL


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        sdi.load_library(str(tmp_path / "libsparse_decode.so"))
