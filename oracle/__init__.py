"""fp64 CPU oracle for the context-sparse decode step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library neither links nor calls it, and the two share no
code.  The arithmetic lives in oracle.c (plain C loops, fp64, OpenMP over
(batch, query head)); this module only marshals numpy arrays.

Functions and the passages they follow (the pages are the context-sparsity
paper, in its Chinese rendering and its German technical summary, and a
sparse-attention survey blog):

* ``scores``  raw q.K^T per cached token: the product inside scaled dot-product
  attention (survey blog, section 1.1).  Pinned by closed forms (one-hot keys,
  integer inputs, shift invariance) in tests/test_oracle_pins.py.
* ``topk``    exact top-k with the lower index winning ties: the "oracle top-k"
  selection of the German summary (section 2, sparsity mechanisms).  Pinned by
  brute force over all subsets on tiny inputs and an independent rank count.
* ``attend``  softmax attention over the selected rows, scale 1/sqrt(128) by
  default: the sparse decode mode of the paper's Fig. 1a with the output form of
  its Theorem 1 (o = V^T a, a a distribution).  Pinned by a direct formula in
  exact rational arithmetic on tiny inputs, uniform-value and uniform-key closed
  forms, the one-hot closed form and k = 1.
* ``dense``   the same over every cached token: the dense mode of Fig. 1a.
  Pinned by the k = N invariant and the closed forms above.
* ``label_scores``  reduced-channel scores for a lightweight indexer (the paper's
  Fig. 1a indexer; the German summary, section 3, costs one with Double Sparsity;
  the Sparse Frontier review, section 3.2, approximate scores from a few key
  dimensions): s~ = sum over a kv head's R listed channels of q_c K_c.  Selection
  is ``topk`` on s~.  Pinned by equality with ``scores`` when the channels are all
  128 (or the keys vanish off the listed channels) and by exact rationals.
* ``quest_summaries`` / ``quest_bounds`` / ``quest_select``  Quest-style page
  selection (the Sparse Frontier review: section 3.5 Table 1, section 7.1, Eq. 10):
  per 16-token page the elementwise min and max of its keys, the bound
  sum_d max(q_d min_d, q_d max_d), and the current page plus the m - 1 other pages
  of highest bound.  Pinned by the box property of min/max, the bound dominating
  every token score of its page (tight for constant pages, closed forms for
  one-signed queries), brute force over page subsets, and m >= pages giving dense.
* ``sample_residual`` / ``attend_sampled``  stochastic index selection (the German
  summary, sections 2 and 3A, vAttention; its estimator is not on the pages, so the
  plain Monte Carlo reading): the top-k set plus s' tokens drawn uniformly with
  replacement from the rest (M tokens), each drawn token weighted M / s' in the
  softmax sums.  Pinned by draws that enumerate the residual (once: weight 1, the
  rest exactly; twice: weight 1/2) giving dense attention, by the residual list
  against a set difference, and by residuals of identical rows, where any draw gives
  the dense output exactly.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DEFAULT_SCALE = 1.0 / math.sqrt(128.0)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP) into oracle/liboracle.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags, _SRC, "-o",
           _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _declare(lib):
    p, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_scores.argtypes = [p, p, p, i32, i32, i32, p, i32, i64, p]
    lib.oracle_topk.argtypes = [p, p, p, i32, i32, i64, i32, p, p]
    lib.oracle_attend.argtypes = [p, p, p, p, i32, i32, i32, p, i32, p, i32, f64, p]
    lib.oracle_dense.argtypes = [p, p, p, p, i32, i32, i32, p, i32, f64, p]
    lib.oracle_label_scores.argtypes = [p, p, p, i32, i32, i32, p, i32, p, i32, i64, p]
    lib.oracle_quest_summaries.argtypes = [p, p, p, i32, i32, i32, p]
    lib.oracle_quest_bounds.argtypes = [p, p, i32, i32, i32, p, i32, p]
    lib.oracle_quest_select.argtypes = [p, p, p, i32, i32, i32, i32, p, p, p]
    lib.oracle_sample_residual.argtypes = [p, p, i32, p, i32, i32, p, p, i32, p, p]
    lib.oracle_attend_sampled.argtypes = [p, p, p, p, i32, i32, i32, p, i32, p, i32, p, i32, p, f64, p]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def load_variant(path: str):
    """Load another build of oracle.c (used by the tests that plant mistakes in it)."""
    return _declare(ctypes.CDLL(path))


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


class Cache:
    """Host view of a paged cache: bf16 bit arrays [pages][Hkv][16][128] + page table."""

    def __init__(self, k_cache, v_cache, page_table, seq_lens, num_kv_heads=None):
        self.k, self.kp = _c(k_cache, np.uint16)
        self.v, self.vp = _c(v_cache, np.uint16)
        self.pt, self.ptp = _c(page_table, np.int32)
        self.sl, self.slp = _c(seq_lens, np.int32)
        self.batch = int(self.pt.shape[0])
        self.max_pages = int(self.pt.shape[1])
        self.num_kv_heads = int(num_kv_heads if num_kv_heads is not None else self.k.shape[1])
        assert self.k.shape[2:] == (16, 128), "cache rows must be [..][16][128]"

    @classmethod
    def of(cls, wl):
        return cls(wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.num_kv_heads)


def scores(cache: Cache, q, lib=None) -> np.ndarray:
    """fp64 scores [B][Hq][n_max] (NaN beyond each sequence's length)."""
    lib = lib or _load()
    q, qp = _c(q, np.uint16)
    hq = q.shape[1]
    n_max = int(cache.sl.max())
    out = np.full((cache.batch, hq, n_max), np.nan)
    lib.oracle_scores(cache.kp, cache.ptp, cache.slp, cache.batch, cache.num_kv_heads, cache.max_pages,
                      qp, hq, n_max, out.ctypes.data_as(ctypes.c_void_p))
    return out


def topk(score_arr, seq_lens, k_per_seq, k_max: int, lib=None):
    """(idx [B][Hq][k_max] int32 ascending then -1, kth-score [B][Hq] fp64)."""
    lib = lib or _load()
    s, sp = _c(score_arr, np.float64)
    sl, slp = _c(seq_lens, np.int32)
    kk, kkp = _c(k_per_seq, np.int32)
    B, hq, n_stride = s.shape
    idx = np.empty((B, hq, k_max), dtype=np.int32)
    kth = np.empty((B, hq), dtype=np.float64)
    lib.oracle_topk(sp, slp, kkp, B, hq, n_stride, k_max, idx.ctypes.data_as(ctypes.c_void_p),
                    kth.ctypes.data_as(ctypes.c_void_p))
    return idx, kth


def attend(cache: Cache, q, idx, scale: float = DEFAULT_SCALE, lib=None) -> np.ndarray:
    """fp64 softmax attention over idx [B][Hq][k_max] (-1 skipped) -> [B][Hq][128]."""
    lib = lib or _load()
    q, qp = _c(q, np.uint16)
    ix, ixp = _c(idx, np.int32)
    B, hq, kmax = ix.shape
    out = np.empty((B, hq, 128), dtype=np.float64)
    lib.oracle_attend(cache.kp, cache.vp, cache.ptp, cache.slp, B, cache.num_kv_heads, cache.max_pages,
                      qp, hq, ixp, kmax, scale, out.ctypes.data_as(ctypes.c_void_p))
    return out


def dense(cache: Cache, q, scale: float = DEFAULT_SCALE, lib=None) -> np.ndarray:
    """fp64 softmax attention over every cached token -> [B][Hq][128]."""
    lib = lib or _load()
    q, qp = _c(q, np.uint16)
    hq = q.shape[1]
    out = np.empty((cache.batch, hq, 128), dtype=np.float64)
    lib.oracle_dense(cache.kp, cache.vp, cache.ptp, cache.slp, cache.batch, cache.num_kv_heads,
                     cache.max_pages, qp, hq, scale, out.ctypes.data_as(ctypes.c_void_p))
    return out


def decode_step(cache: Cache, q, k_per_seq, k_max: int, scale: float = DEFAULT_SCALE, lib=None):
    """The whole sparse step: scores -> exact top-k -> attend.  Returns (idx, kth, scores, out)."""
    s = scores(cache, q, lib=lib)
    idx, kth = topk(s, cache.sl, k_per_seq, k_max, lib=lib)
    out = attend(cache, q, idx, scale, lib=lib)
    return idx, kth, s, out


def quest_summaries(cache: Cache, lib=None) -> np.ndarray:
    """Per logical page [B][max_pages][Hkv][2][128] fp64: [0] the min, [1] the max of the
    page's cached key rows (NaN for pages past the sequence)."""
    lib = lib or _load()
    out = np.full((cache.batch, cache.max_pages, cache.num_kv_heads, 2, 128), np.nan)
    lib.oracle_quest_summaries(cache.kp, cache.ptp, cache.slp, cache.batch, cache.num_kv_heads, cache.max_pages,
                               out.ctypes.data_as(ctypes.c_void_p))
    return out


def quest_bounds(summ, seq_lens, q, lib=None) -> np.ndarray:
    """U [B][Hq][max_pages] fp64, U = sum_d max(q_d min_d, q_d max_d) (NaN past the sequence)."""
    lib = lib or _load()
    sm, smp = _c(summ, np.float64)
    sl, slp = _c(seq_lens, np.int32)
    q, qp = _c(q, np.uint16)
    B, max_pages, hkv = sm.shape[:3]
    hq = q.shape[1]
    out = np.full((B, hq, max_pages), np.nan)
    lib.oracle_quest_bounds(smp, slp, B, hkv, max_pages, qp, hq, out.ctypes.data_as(ctypes.c_void_p))
    return out


def quest_select(u, seq_lens, m_per_seq, m_max: int, lib=None):
    """(pages [B][Hq][m_max], tokens [B][Hq][16 m_max], threshold [B][Hq]): the current
    page plus the m - 1 other pages of highest bound (lower page first on ties)."""
    lib = lib or _load()
    uu, up = _c(u, np.float64)
    sl, slp = _c(seq_lens, np.int32)
    mm, mmp = _c(m_per_seq, np.int32)
    B, hq, max_pages = uu.shape
    pages = np.empty((B, hq, m_max), dtype=np.int32)
    toks = np.empty((B, hq, 16 * m_max), dtype=np.int32)
    thr = np.empty((B, hq), dtype=np.float64)
    lib.oracle_quest_select(up, slp, mmp, B, hq, max_pages, m_max, pages.ctypes.data_as(ctypes.c_void_p),
                            toks.ctypes.data_as(ctypes.c_void_p), thr.ctypes.data_as(ctypes.c_void_p))
    return pages, toks, thr


def label_scores(cache: Cache, q, channels, lib=None) -> np.ndarray:
    """fp64 reduced-channel scores [B][Hq][n_max]: sum over channels[g] (int32 [Hkv][R])
    of q_c K_c, in the listed order (NaN beyond each sequence's length)."""
    lib = lib or _load()
    q, qp = _c(q, np.uint16)
    ch, chp = _c(channels, np.int32)
    hq = q.shape[1]
    n_max = int(cache.sl.max())
    out = np.full((cache.batch, hq, n_max), np.nan)
    lib.oracle_label_scores(cache.kp, cache.ptp, cache.slp, cache.batch, cache.num_kv_heads, cache.max_pages,
                            qp, hq, chp, ch.shape[1], n_max, out.ctypes.data_as(ctypes.c_void_p))
    return out


def sample_residual(idx, k_per_seq, seq_lens, draws, s_per_seq, lib=None):
    """(sample [B][Hq][s_max] int32, weight [B][Hq] fp64): draw t of row (b, h) is the
    residual token of rank floor(draws[b,h,t] M / 2^32), M = N_b - |kept set|; weight
    M / s'_b, s'_b = min(s_b, s_max) (0 and -1 entries when nothing is drawn)."""
    lib = lib or _load()
    ix, ixp = _c(idx, np.int32)
    kk, kkp = _c(k_per_seq, np.int32)
    sl, slp = _c(seq_lens, np.int32)
    dr, drp = _c(draws, np.uint32)
    ss, ssp = _c(s_per_seq, np.int32)
    B, hq, k_max = ix.shape
    s_max = dr.shape[2]
    sample = np.empty((B, hq, s_max), dtype=np.int32)
    weight = np.empty((B, hq), dtype=np.float64)
    lib.oracle_sample_residual(ixp, kkp, k_max, slp, B, hq, drp, ssp, s_max, sample.ctypes.data_as(ctypes.c_void_p),
                               weight.ctypes.data_as(ctypes.c_void_p))
    return sample, weight


def attend_sampled(cache: Cache, q, idx, sample, weight, scale: float = DEFAULT_SCALE, lib=None) -> np.ndarray:
    """fp64 stochastic estimate [B][Hq][128]: softmax sums over idx (weight 1) and
    sample (weight[b,h] per entry), -1 entries skipped."""
    lib = lib or _load()
    q, qp = _c(q, np.uint16)
    ix, ixp = _c(idx, np.int32)
    sm, smp = _c(sample, np.int32)
    w, wp = _c(weight, np.float64)
    B, hq, k_max = ix.shape
    out = np.empty((B, hq, 128), dtype=np.float64)
    lib.oracle_attend_sampled(cache.kp, cache.vp, cache.ptp, cache.slp, B, cache.num_kv_heads, cache.max_pages,
                              qp, hq, ixp, k_max, smp, sm.shape[2], wp, scale, out.ctypes.data_as(ctypes.c_void_p))
    return out
