"""Context-sparse decode on MI355X (gfx950): exact top-k indexer, sparse gather-attend
and a dense decode reference, over a paged bf16 KV cache.

This module is a thin ctypes binding over the C ABI in include/sparse_decode.h
(libsparse_decode.so, built in-tree by build.py).  It only marshals arguments:
torch tensors supply device pointers and the current HIP stream; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_decode.so")

HEAD_DIM = 128
PAGE_SIZE = 16
DEFAULT_SCALE = 1.0 / math.sqrt(HEAD_DIM)

SDI_OK, SDI_ERR_NULL, SDI_ERR_SHAPE, SDI_ERR_K, SDI_ERR_WORKSPACE, SDI_ERR_HIP = 0, -1, -2, -3, -4, -5
SDI_ERR_TOO_LARGE = -6

EXPORTS = (
    "sparse_decode_index_topk", "sparse_decode_index_topk_workspace",
    "sparse_decode_attend", "sparse_decode_attend_workspace", "sparse_decode_attend_noalloc",
    "dense_decode", "dense_decode_workspace", "sparse_decode_strerror",
    "sparse_decode_quest_summary_bytes", "sparse_decode_quest_summarize",
    "sparse_decode_quest_select", "sparse_decode_quest_select_workspace",
    "sparse_decode_label_bytes", "sparse_decode_label_build", "sparse_decode_label_index_topk",
    "sparse_decode_sample_residual", "sparse_decode_attend_sampled", "sparse_decode_attend_sampled_workspace",
)


class SdiKV(ctypes.Structure):
    """Mirror of struct sdi_kv."""
    _fields_ = [
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("n_max", ctypes.c_int32),
    ]


class SparseDecodeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} (status {code})")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libsparse_decode.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python {os.path.join(HERE, 'build.py')}`")
    lib = ctypes.CDLL(path)
    p, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    kvp = ctypes.POINTER(SdiKV)
    lib.sparse_decode_index_topk.argtypes = [kvp, p, i32, p, i32, p, p, sz, p]
    lib.sparse_decode_index_topk.restype = ctypes.c_int
    lib.sparse_decode_index_topk_workspace.argtypes = [kvp, i32, i32]
    lib.sparse_decode_index_topk_workspace.restype = sz
    lib.sparse_decode_attend.argtypes = [kvp, p, i32, p, p, i32, f32, p, p, sz, p]
    lib.sparse_decode_attend.restype = ctypes.c_int
    lib.sparse_decode_attend_workspace.argtypes = [kvp, i32, i32]
    lib.sparse_decode_attend_workspace.restype = sz
    lib.sparse_decode_attend_noalloc.argtypes = [kvp, p, i32, p, p, i32, f32, p, p]
    lib.sparse_decode_attend_noalloc.restype = ctypes.c_int
    lib.dense_decode.argtypes = [kvp, p, i32, f32, p, p, sz, p]
    lib.dense_decode.restype = ctypes.c_int
    lib.dense_decode_workspace.argtypes = [kvp, i32]
    lib.dense_decode_workspace.restype = sz
    lib.sparse_decode_label_bytes.argtypes = [kvp]
    lib.sparse_decode_label_bytes.restype = sz
    lib.sparse_decode_label_build.argtypes = [kvp, p, p, i32, p]
    lib.sparse_decode_label_build.restype = ctypes.c_int
    lib.sparse_decode_label_index_topk.argtypes = [kvp, p, i32, p, p, p, i32, p, p, sz, p]
    lib.sparse_decode_label_index_topk.restype = ctypes.c_int
    lib.sparse_decode_quest_summary_bytes.argtypes = [kvp]
    lib.sparse_decode_quest_summary_bytes.restype = sz
    lib.sparse_decode_quest_summarize.argtypes = [kvp, p, i32, p]
    lib.sparse_decode_quest_summarize.restype = ctypes.c_int
    lib.sparse_decode_quest_select.argtypes = [kvp, p, i32, p, p, i32, p, p, sz, p]
    lib.sparse_decode_quest_select.restype = ctypes.c_int
    lib.sparse_decode_quest_select_workspace.argtypes = [kvp, i32, i32]
    lib.sparse_decode_quest_select_workspace.restype = sz
    lib.sparse_decode_sample_residual.argtypes = [kvp, i32, p, p, i32, p, p, i32, p, p, p]
    lib.sparse_decode_sample_residual.restype = ctypes.c_int
    lib.sparse_decode_attend_sampled.argtypes = [kvp, p, i32, p, p, i32, p, p, p, i32, f32, p, p, sz, p]
    lib.sparse_decode_attend_sampled.restype = ctypes.c_int
    lib.sparse_decode_attend_sampled_workspace.argtypes = [kvp, i32, i32, i32]
    lib.sparse_decode_attend_sampled_workspace.restype = sz
    lib.sparse_decode_strerror.argtypes = [ctypes.c_int]
    lib.sparse_decode_strerror.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().sparse_decode_strerror(int(code)).decode()


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(t, name, dtype, ndim, shape=None, min_len=None):
    """Type, rank, shape and layout of one tensor argument.  `shape` lists the expected
    sizes (None = any); `min_len` is a lower bound on a 1-d tensor's length.  The C ABI
    cannot see tensor sizes, so a mismatch caught here is what stops a kernel from
    reading or writing past a buffer.  Every entry point checks all shapes first and the
    devices last (_on_device)."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None:
        for got, want in zip(t.shape, shape):
            if want is not None and int(got) != int(want):
                want_s = tuple("*" if w is None else int(w) for w in shape)
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want_s}")
    if min_len is not None and int(t.shape[0]) < int(min_len):
        raise ValueError(f"{name} holds {int(t.shape[0])} entries, needs at least {int(min_len)} (one per sequence)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _check_q(kv, q):
    """q must be bf16 [batch][Hq][128] with Hq a multiple of the kv heads; returns Hq."""
    import torch
    _check(q, "q", torch.bfloat16, 3, (kv.batch, None, HEAD_DIM))
    hq = int(q.shape[1])
    if hq < 1 or hq % kv.num_kv_heads != 0:
        raise ValueError(f"q has {hq} heads, not a positive multiple of the cache's {kv.num_kv_heads} kv heads")
    return hq


def _check_counts(kv, t, name):
    import torch
    if t is not None:
        _check(t, name, torch.int32, 1, min_len=kv.batch)


class PagedKV:
    """A paged bf16 KV cache on the device: k/v [pages][Hkv][16][128] (bf16), page_table
    [B][max_pages] int32, seq_lens [B] int32, plus the host value n_max = max(seq_lens)."""

    def __init__(self, k_cache, v_cache, page_table, seq_lens, n_max: Optional[int] = None):
        import torch
        _check(k_cache, "k_cache", torch.bfloat16, 4, (None, None, PAGE_SIZE, HEAD_DIM))
        if v_cache is not None:
            _check(v_cache, "v_cache", torch.bfloat16, 4, tuple(k_cache.shape))
        _check(page_table, "page_table", torch.int32, 2)
        _check(seq_lens, "seq_lens", torch.int32, 1, (page_table.shape[0],))
        _on_device(k_cache=k_cache, v_cache=v_cache, page_table=page_table, seq_lens=seq_lens)
        self.k_cache, self.v_cache, self.page_table, self.seq_lens = k_cache, v_cache, page_table, seq_lens
        self.n_max = int(seq_lens.max().item()) if n_max is None else int(n_max)
        if self.n_max > int(page_table.shape[1]) * PAGE_SIZE:
            raise ValueError(f"n_max {self.n_max} needs more than the page table's {int(page_table.shape[1])} pages")

    @property
    def batch(self) -> int:
        return int(self.page_table.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[1])

    def struct(self) -> SdiKV:
        k = self.k_cache
        return SdiKV(_ptr(k), _ptr(self.v_cache), _ptr(self.page_table), _ptr(self.seq_lens),
                     int(self.page_table.shape[0]), int(k.shape[1]), int(k.shape[3]), int(k.shape[2]),
                     int(self.page_table.shape[1]), int(k.shape[0]), self.n_max)


def index_topk_workspace_bytes(kv: PagedKV, num_q_heads: int, k_max: int) -> int:
    s = kv.struct()
    return int(load_library().sparse_decode_index_topk_workspace(ctypes.byref(s), num_q_heads, k_max))


def attend_workspace_bytes(kv: PagedKV, num_q_heads: int, k_max: int) -> int:
    s = kv.struct()
    return int(load_library().sparse_decode_attend_workspace(ctypes.byref(s), num_q_heads, k_max))


def attend_sampled_workspace_bytes(kv: PagedKV, num_q_heads: int, k_max: int, s_max: int) -> int:
    s = kv.struct()
    return int(load_library().sparse_decode_attend_sampled_workspace(ctypes.byref(s), num_q_heads, k_max, s_max))


def dense_workspace_bytes(kv: PagedKV, num_q_heads: int) -> int:
    s = kv.struct()
    return int(load_library().dense_decode_workspace(ctypes.byref(s), num_q_heads))


def _workspace(nbytes: int, device, workspace):
    import torch
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def index_topk(kv: PagedKV, q, k_per_seq, k_max: int, idx_out=None, workspace=None, stream=None):
    """Exact top-k per (b, query head): int32 [B][Hq][k_max], ascending, -1 padded."""
    import torch
    hq = _check_q(kv, q)
    _check(k_per_seq, "k_per_seq", torch.int32, 1, min_len=kv.batch)
    B = kv.batch
    if idx_out is None:
        idx_out = torch.empty((B, hq, k_max), dtype=torch.int32, device=q.device)
    _check(idx_out, "idx_out", torch.int32, 3, (B, hq, k_max))
    _on_device(q=q, k_per_seq=k_per_seq, idx_out=idx_out)
    s = kv.struct()
    lib = load_library()
    ws = _workspace(lib.sparse_decode_index_topk_workspace(ctypes.byref(s), hq, k_max), q.device, workspace)
    rc = lib.sparse_decode_index_topk(ctypes.byref(s), _ptr(q), hq, _ptr(k_per_seq), k_max, _ptr(idx_out),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_index_topk")
    return idx_out


def attend(kv: PagedKV, q, idx, k_per_seq=None, softmax_scale: float = DEFAULT_SCALE, out=None,
           workspace=None, stream=None):
    """Softmax attention over the listed rows: fp32 [B][Hq][128]."""
    import torch
    hq = _check_q(kv, q)
    B = kv.batch
    _check(idx, "idx", torch.int32, 3, (B, hq, None))
    _check_counts(kv, k_per_seq, "k_per_seq")
    k_max = int(idx.shape[2])
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.float32, 3, (B, hq, HEAD_DIM))
    _on_device(q=q, idx=idx, k_per_seq=k_per_seq, out=out)
    s = kv.struct()
    lib = load_library()
    ws = _workspace(lib.sparse_decode_attend_workspace(ctypes.byref(s), hq, k_max), q.device, workspace)
    rc = lib.sparse_decode_attend(ctypes.byref(s), _ptr(q), hq, _ptr(idx), _ptr(k_per_seq), k_max,
                                  float(softmax_scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_attend")
    return out


def attend_noalloc(kv: PagedKV, q, idx, k_per_seq=None, softmax_scale: float = DEFAULT_SCALE, out=None,
                   stream=None):
    """attend() without a workspace (sparse_decode_attend_noalloc): split rows keep their
    partials in the library's fixed 32 MiB per-GPU scratch.  With out given, nothing is
    allocated; calls that overlap on one GPU race."""
    import torch
    hq = _check_q(kv, q)
    B = kv.batch
    _check(idx, "idx", torch.int32, 3, (B, hq, None))
    _check_counts(kv, k_per_seq, "k_per_seq")
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.float32, 3, (B, hq, HEAD_DIM))
    _on_device(q=q, idx=idx, k_per_seq=k_per_seq, out=out)
    s = kv.struct()
    rc = load_library().sparse_decode_attend_noalloc(ctypes.byref(s), _ptr(q), hq, _ptr(idx), _ptr(k_per_seq),
                                                     int(idx.shape[2]), float(softmax_scale), _ptr(out),
                                                     _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_attend_noalloc")
    return out


def dense(kv: PagedKV, q, softmax_scale: float = DEFAULT_SCALE, out=None, workspace=None, stream=None):
    """Softmax attention over every cached token: fp32 [B][Hq][128]."""
    import torch
    hq = _check_q(kv, q)
    B = kv.batch
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.float32, 3, (B, hq, HEAD_DIM))
    _on_device(q=q, out=out)
    s = kv.struct()
    lib = load_library()
    ws = _workspace(lib.dense_decode_workspace(ctypes.byref(s), hq), q.device, workspace)
    rc = lib.dense_decode(ctypes.byref(s), _ptr(q), hq, float(softmax_scale), _ptr(out), _ptr(ws),
                          ws.numel() * ws.element_size(), _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "dense_decode")
    return out


def decode_step(kv: PagedKV, q, k_per_seq, k_max: int, softmax_scale: float = DEFAULT_SCALE,
                idx_out=None, out=None, index_ws=None, attend_ws=None, stream=None):
    """One sparse decode step: exact top-k, then attend over the selected rows."""
    idx = index_topk(kv, q, k_per_seq, k_max, idx_out=idx_out, workspace=index_ws, stream=stream)
    return idx, attend(kv, q, idx, k_per_seq, softmax_scale, out=out, workspace=attend_ws, stream=stream)


def quest_summarize(kv: PagedKV, summary=None, current_pages_only: bool = False, stream=None):
    """Page min/max key summaries, bf16 [num_pages][Hkv][2][128] (min row, max row).
    With current_pages_only, only each sequence's last page is (re)written."""
    import torch
    s = kv.struct()
    lib = load_library()
    if summary is None:
        summary = torch.empty((s.num_pages, s.num_kv_heads, 2, HEAD_DIM), dtype=torch.bfloat16,
                              device=kv.k_cache.device)
    _check(summary, "summary", torch.bfloat16, 4, (s.num_pages, s.num_kv_heads, 2, HEAD_DIM))
    _on_device(summary=summary)
    rc = lib.sparse_decode_quest_summarize(ctypes.byref(s), _ptr(summary), 1 if current_pages_only else 0,
                                           _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_quest_summarize")
    return summary


def quest_select(kv: PagedKV, q, summary, pages_per_seq, pages_max: int, idx_out=None, workspace=None,
                 stream=None):
    """Current page plus the highest-bound pages per (b, query head): token indices
    int32 [B][Hq][16 pages_max] (page by page, -1 past N_b or past the selection)."""
    import torch
    hq = _check_q(kv, q)
    _check(pages_per_seq, "pages_per_seq", torch.int32, 1, min_len=kv.batch)
    B = kv.batch
    s = kv.struct()
    _check(summary, "summary", torch.bfloat16, 4, (s.num_pages, s.num_kv_heads, 2, HEAD_DIM))
    if idx_out is None:
        idx_out = torch.empty((B, hq, 16 * pages_max), dtype=torch.int32, device=q.device)
    _check(idx_out, "idx_out", torch.int32, 3, (B, hq, 16 * pages_max))
    _on_device(q=q, pages_per_seq=pages_per_seq, summary=summary, idx_out=idx_out)
    lib = load_library()
    ws = _workspace(lib.sparse_decode_quest_select_workspace(ctypes.byref(s), hq, pages_max), q.device, workspace)
    rc = lib.sparse_decode_quest_select(ctypes.byref(s), _ptr(q), hq, _ptr(summary), _ptr(pages_per_seq),
                                        pages_max, _ptr(idx_out), _ptr(ws), ws.numel() * ws.element_size(),
                                        _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_quest_select")
    return idx_out


def label_build(kv: PagedKV, channels, labels=None, current_pages_only: bool = False, stream=None):
    """Label rows bf16 [num_pages][Hkv][16][16]: channels (int32 [Hkv][16], device) of
    every cached key row.  With current_pages_only, only each sequence's last page."""
    import torch
    s = kv.struct()
    _check(channels, "channels", torch.int32, 2, (s.num_kv_heads, 16))
    lib = load_library()
    if labels is None:
        labels = torch.empty((s.num_pages, s.num_kv_heads, 16, 16), dtype=torch.bfloat16, device=kv.k_cache.device)
    _check(labels, "labels", torch.bfloat16, 4, (s.num_pages, s.num_kv_heads, 16, 16))
    _on_device(channels=channels, labels=labels)
    rc = lib.sparse_decode_label_build(ctypes.byref(s), _ptr(channels), _ptr(labels),
                                       1 if current_pages_only else 0, _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_label_build")
    return labels


def label_index_topk(kv: PagedKV, q, labels, channels, k_per_seq, k_max: int, idx_out=None, workspace=None,
                     stream=None):
    """Top-k per (b, query head) of the reduced-channel scores: int32 [B][Hq][k_max]."""
    import torch
    hq = _check_q(kv, q)
    _check(k_per_seq, "k_per_seq", torch.int32, 1, min_len=kv.batch)
    B = kv.batch
    s = kv.struct()
    _check(channels, "channels", torch.int32, 2, (s.num_kv_heads, 16))
    _check(labels, "labels", torch.bfloat16, 4, (s.num_pages, s.num_kv_heads, 16, 16))
    if idx_out is None:
        idx_out = torch.empty((B, hq, k_max), dtype=torch.int32, device=q.device)
    _check(idx_out, "idx_out", torch.int32, 3, (B, hq, k_max))
    _on_device(q=q, k_per_seq=k_per_seq, channels=channels, labels=labels, idx_out=idx_out)
    lib = load_library()
    ws = _workspace(lib.sparse_decode_index_topk_workspace(ctypes.byref(s), hq, k_max), q.device, workspace)
    rc = lib.sparse_decode_label_index_topk(ctypes.byref(s), _ptr(q), hq, _ptr(labels), _ptr(channels),
                                            _ptr(k_per_seq), k_max, _ptr(idx_out), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_label_index_topk")
    return idx_out


def sample_residual(kv: PagedKV, idx, k_per_seq, draws, s_per_seq, sample_out=None, weight_out=None, stream=None):
    """Uniform draws from the tokens a top-k row left out: (sample int32 [B][Hq][s_max],
    weight fp32 [B][Hq]).  draws: 32-bit random numbers [B][Hq][s_max] (uint32, or
    their bits in int32)."""
    import torch
    _check(idx, "idx", torch.int32, 3, (kv.batch, None, None))
    _check(k_per_seq, "k_per_seq", torch.int32, 1, min_len=kv.batch)
    _check(s_per_seq, "s_per_seq", torch.int32, 1, min_len=kv.batch)
    B, hq, k_max = (int(x) for x in idx.shape)
    if hq < 1 or hq % kv.num_kv_heads != 0:
        raise ValueError(f"idx has {hq} heads, not a positive multiple of the cache's {kv.num_kv_heads} kv heads")
    if draws.dtype not in (torch.int32, torch.uint32) or draws.dim() != 3 or not draws.is_contiguous():
        raise ValueError("draws must be a contiguous 3-d int32 or uint32 tensor")
    if tuple(draws.shape[:2]) != (B, hq):
        raise ValueError(f"draws has shape {tuple(draws.shape)}, expected ({B}, {hq}, *)")
    s_max = int(draws.shape[2])
    if sample_out is None:
        sample_out = torch.empty((B, hq, s_max), dtype=torch.int32, device=idx.device)
    if weight_out is None:
        weight_out = torch.empty((B, hq), dtype=torch.float32, device=idx.device)
    _check(sample_out, "sample_out", torch.int32, 3, (B, hq, s_max))
    _check(weight_out, "weight_out", torch.float32, 2, (B, hq))
    _on_device(idx=idx, k_per_seq=k_per_seq, s_per_seq=s_per_seq, draws=draws, sample_out=sample_out,
               weight_out=weight_out)
    s = kv.struct()
    rc = load_library().sparse_decode_sample_residual(ctypes.byref(s), hq, _ptr(idx), _ptr(k_per_seq), k_max,
                                                      _ptr(draws), _ptr(s_per_seq), s_max, _ptr(sample_out),
                                                      _ptr(weight_out), _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_sample_residual")
    return sample_out, weight_out


def attend_sampled(kv: PagedKV, q, idx, k_per_seq, sample, sample_weight, s_per_seq=None,
                   softmax_scale: float = DEFAULT_SCALE, out=None, workspace=None, stream=None):
    """The stochastic estimate: softmax sums over idx (weight 1) and sample (weight
    sample_weight[b, h] per entry): fp32 [B][Hq][128]."""
    import torch
    hq = _check_q(kv, q)
    B = kv.batch
    _check(idx, "idx", torch.int32, 3, (B, hq, None))
    _check_counts(kv, k_per_seq, "k_per_seq")
    _check_counts(kv, s_per_seq, "s_per_seq")
    _check(sample, "sample", torch.int32, 3, (B, hq, None))
    _check(sample_weight, "sample_weight", torch.float32, 2, (B, hq))
    k_max, s_max = int(idx.shape[2]), int(sample.shape[2])
    if out is None:
        out = torch.empty((B, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.float32, 3, (B, hq, HEAD_DIM))
    _on_device(q=q, idx=idx, k_per_seq=k_per_seq, s_per_seq=s_per_seq, sample=sample,
               sample_weight=sample_weight, out=out)
    s = kv.struct()
    lib = load_library()
    ws = _workspace(lib.sparse_decode_attend_sampled_workspace(ctypes.byref(s), hq, k_max, s_max), q.device,
                    workspace)
    rc = lib.sparse_decode_attend_sampled(ctypes.byref(s), _ptr(q), hq, _ptr(idx), _ptr(k_per_seq), k_max,
                                          _ptr(sample), _ptr(sample_weight), _ptr(s_per_seq), s_max,
                                          float(softmax_scale), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                          _stream(stream))
    if rc != SDI_OK:
        raise SparseDecodeError(rc, "sparse_decode_attend_sampled")
    return out
