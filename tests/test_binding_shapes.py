"""The Python binding checks tensor shapes against the cache before any C call: the C ABI
sees only pointers, so a tensor of the wrong size would otherwise send a kernel past a
buffer.  CPU tensors are used, so every check below must fire before the device check
(which would reject them with a different message) and before anything is launched."""
import pytest

torch = pytest.importorskip("torch")

import sparse_attention_decode_index_amd as sdi

B, HKV, HQ, PAGES, MAXP = 2, 2, 8, 40, 10


class CpuKV(sdi.PagedKV):
    """A PagedKV over host tensors (the constructor's device check skipped)."""

    def __init__(self):
        self.k_cache = torch.zeros((PAGES, HKV, 16, 128), dtype=torch.bfloat16)
        self.v_cache = torch.zeros_like(self.k_cache)
        self.page_table = torch.zeros((B, MAXP), dtype=torch.int32)
        self.seq_lens = torch.full((B,), 150, dtype=torch.int32)
        self.n_max = 150


def bf16(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def shape_error(fn, *a, **kw):
    with pytest.raises(ValueError) as e:
        fn(*a, **kw)
    msg = str(e.value)
    assert "device tensor" not in msg, msg        # the shape check came first
    return msg


@pytest.fixture
def kv():
    return CpuKV()


def test_paged_kv_rejects_bad_cache_shapes():
    pt, sl = i32(B, MAXP), i32(B)
    shape_error(sdi.PagedKV, bf16(PAGES, HKV, 8, 128), None, pt, sl, n_max=1)        # page size 8
    shape_error(sdi.PagedKV, bf16(PAGES, HKV, 16, 64), None, pt, sl, n_max=1)        # head_dim 64
    shape_error(sdi.PagedKV, bf16(PAGES, HKV, 16, 128), bf16(PAGES, 1, 16, 128), pt, sl, n_max=1)
    shape_error(sdi.PagedKV, bf16(PAGES, HKV, 16, 128), None, pt, i32(B + 1), n_max=1)  # one length per row


def test_q_must_match_the_batch_and_heads(kv):
    kps = i32(B)
    shape_error(sdi.index_topk, kv, bf16(B + 1, HQ, 128), kps, 5)
    shape_error(sdi.index_topk, kv, bf16(B, HQ, 64), kps, 5)
    shape_error(sdi.index_topk, kv, bf16(B, 7, 128), kps, 5)                       # not a multiple of Hkv
    shape_error(sdi.dense, kv, bf16(B - 1, HQ, 128))
    shape_error(sdi.attend, kv, bf16(B, HQ, 100), i32(B, HQ, 5))


def test_index_topk_shapes(kv):
    q = bf16(B, HQ, 128)
    shape_error(sdi.index_topk, kv, q, i32(B - 1), 5)                              # k_per_seq too short
    shape_error(sdi.index_topk, kv, q, i32(B), 5, idx_out=i32(B, HQ, 4))           # idx_out too small
    shape_error(sdi.index_topk, kv, q, i32(B), 5, idx_out=i32(B, HQ - 1, 5))


def test_attend_and_dense_shapes(kv):
    q = bf16(B, HQ, 128)
    shape_error(sdi.attend, kv, q, i32(B, HQ - 2, 5))
    shape_error(sdi.attend, kv, q, i32(B, HQ, 5), i32(B - 1))
    shape_error(sdi.attend, kv, q, i32(B, HQ, 5), out=f32(B, HQ, 64))
    shape_error(sdi.dense, kv, q, out=f32(B, HQ + 1, 128))


def test_quest_shapes(kv):
    q = bf16(B, HQ, 128)
    good = bf16(PAGES, HKV, 2, 128)
    shape_error(sdi.quest_summarize, kv, bf16(PAGES - 1, HKV, 2, 128))
    shape_error(sdi.quest_select, kv, q, bf16(PAGES, HKV, 1, 128), i32(B), 3)      # summary shape
    shape_error(sdi.quest_select, kv, q, good, i32(B - 1), 3)                      # pages_per_seq too short
    shape_error(sdi.quest_select, kv, q, good, i32(B), 3, idx_out=i32(B, HQ, 47))  # needs 16 * 3 entries


def test_label_shapes(kv):
    q = bf16(B, HQ, 128)
    labels = bf16(PAGES, HKV, 16, 16)
    shape_error(sdi.label_build, kv, i32(HKV, 8))                                  # 16 channels per kv head
    shape_error(sdi.label_build, kv, i32(HKV + 1, 16))
    shape_error(sdi.label_build, kv, i32(HKV, 16), bf16(PAGES, HKV, 16, 8))
    shape_error(sdi.label_index_topk, kv, q, labels, i32(HKV, 15), i32(B), 5)
    shape_error(sdi.label_index_topk, kv, q, bf16(PAGES - 1, HKV, 16, 16), i32(HKV, 16), i32(B), 5)
    shape_error(sdi.label_index_topk, kv, q, labels, i32(HKV, 16), i32(B - 1), 5)
    shape_error(sdi.label_index_topk, kv, q, labels, i32(HKV, 16), i32(B), 5, idx_out=i32(B, HQ, 6))


def test_sample_shapes(kv):
    idx = i32(B, HQ, 5)
    draws = torch.zeros((B, HQ, 7), dtype=torch.int32)
    shape_error(sdi.sample_residual, kv, i32(B + 1, HQ, 5), i32(B), draws, i32(B))
    shape_error(sdi.sample_residual, kv, idx, i32(B - 1), draws, i32(B))
    shape_error(sdi.sample_residual, kv, idx, i32(B), draws, i32(B - 1))
    shape_error(sdi.sample_residual, kv, i32(B, 5, 5), i32(B), torch.zeros((B, 5, 7), dtype=torch.int32), i32(B))
    shape_error(sdi.sample_residual, kv, idx, i32(B), torch.zeros((B, HQ - 1, 7), dtype=torch.int32), i32(B))
    shape_error(sdi.sample_residual, kv, idx, i32(B), draws, i32(B), sample_out=i32(B, HQ, 6))
    shape_error(sdi.sample_residual, kv, idx, i32(B), draws, i32(B), weight_out=f32(B, HQ + 1))
    q = bf16(B, HQ, 128)
    shape_error(sdi.attend_sampled, kv, q, idx, i32(B), i32(B, HQ - 2, 7), f32(B, HQ))
    shape_error(sdi.attend_sampled, kv, q, idx, i32(B), i32(B, HQ, 7), f32(B, HQ - 1))
    shape_error(sdi.attend_sampled, kv, q, idx, i32(B), i32(B, HQ, 7), f32(B, HQ), s_per_seq=i32(1))
    shape_error(sdi.attend_sampled, kv, q, idx, i32(B), i32(B, HQ, 7), f32(B, HQ), out=f32(B, HQ, 127))
