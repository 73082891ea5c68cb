"""Seeded synthetic decode workloads: bf16 queries and a paged bf16 KV cache.

This module builds inputs only.  It holds none of the attention method's
arithmetic (no scores, no selection, no softmax), so both the CPU oracle and
the GPU library can consume what it produces without sharing code.

Shapes follow the context-sparse decode workloads: head_dim 128, page size 16,
GQA with contiguous groups, per-step cache growth.  Value recipes:

* q, K, V ~ N(0, 1), drawn per element from a counter-based generator keyed by
  (seed, tensor, step, batch row, head) and the element's logical position, so
  the logical contents do not depend on the physical page layout.
* planted keys: at seeded distinct positions of each (b, kv head), a key along
  the unit vector of the sum of that group's queries, times sqrt(128), plus
  0.25 * N(0, 1) noise (raw score about 64 against about 23 at the 50x cut).
* outlier channels: seeded channels of each (b, kv head) whose K values are
  2 * Student-t(3) instead of N(0, 1) (heavy-tailed keys).
* page tables: identity ("contiguous"), a seeded permutation of the pool
  ("shuffled"), or a pool 1.25x the need with a seeded free list dealt
  round-robin across sequences, holes left unused and growth pages taken from
  the free list ("fragmented").
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsdi_synth.so")
_lib = None

# tensor ids used in stream tags
T_Q, T_K, T_V, T_PLANT, T_POS, T_CHAN, T_PAGES, T_LENS = 1, 2, 3, 4, 5, 6, 7, 8

HEAD_DIM = 128
PAGE_SIZE = 16


def build(verbose: bool = False) -> str:
    """Compile the generator with gcc (OpenMP) into synth/libsdi_synth.so."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, i32, u32, f32, p = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                  ctypes.c_float, ctypes.c_void_p)
    lib.synth_tag.restype = u64
    lib.synth_tag.argtypes = [u32, u32, u32, u32]
    lib.synth_u64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, f32, p]
    lib.synth_normal_f64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_round_bf16.argtypes = [p, i64, p]
    lib.synth_fill_kv_paged.argtypes = [u64, u32, i32, i32, i32, i32, i32, p, p, p, p, f32, p]
    lib.synth_kv_rows.argtypes = [u64, u32, i32, i32, i32, p, p, f32, p]
    lib.synth_queries.argtypes = [u64, u32, i32, i32, i32, p]
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def tag(tensor: int, step: int = 0, b: int = 0, head: int = 0) -> int:
    return int(_load().synth_tag(tensor, step, b, head))


def u64(seed: int, tensor_tag: int, n: int, ctr0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_u64(seed, tensor_tag, ctr0, n, _ptr(out))
    return out


def permutation(seed: int, tensor_tag: int, n: int) -> np.ndarray:
    """Seeded permutation of range(n) (argsort of n independent 64-bit draws)."""
    return np.argsort(u64(seed, tensor_tag, n), kind="stable").astype(np.int64)


def normal_f64(seed: int, tensor_tag: int, n: int, ctr0: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(seed, tensor_tag, ctr0, n, _ptr(out))
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_round_bf16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (test/bench convenience)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 bit patterns (nearest even)."""
    return round_bf16(np.asarray(x, dtype=np.float64))


# ---- k rules ---------------------------------------------------------------------------------

def k_half_up(ratio: int) -> Callable[[np.ndarray], np.ndarray]:
    """k = N / ratio rounded half up (4096/50 -> 82, 32768/50 -> 655, 131072/20 -> 6554)."""
    def rule(n):
        n = np.asarray(n, dtype=np.int64)
        return ((2 * n + ratio) // (2 * ratio)).astype(np.int32)
    rule.__name__ = f"round(N/{ratio})"
    return rule


def k_ceil(ratio: int) -> Callable[[np.ndarray], np.ndarray]:
    """k = ceil(N / ratio)."""
    def rule(n):
        n = np.asarray(n, dtype=np.int64)
        return ((n + ratio - 1) // ratio).astype(np.int32)
    rule.__name__ = f"ceil(N/{ratio})"
    return rule


def k_fixed(k: int) -> Callable[[np.ndarray], np.ndarray]:
    def rule(n):
        return np.full(np.shape(n), k, dtype=np.int32)
    rule.__name__ = f"k={k}"
    return rule


# ---- workload --------------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: np.ndarray          # int32 [B], current context lengths
    capacity: np.ndarray          # int32 [B], context after all planned growth steps
    page_table: np.ndarray        # int32 [B][max_pages]
    num_pages: int
    k_cache: np.ndarray           # uint16 (bf16 bits) [P][Hkv][16][128]
    v_cache: np.ndarray
    q: np.ndarray                 # uint16 [B][Hq][128], queries of the current step
    k_rule: Callable[[np.ndarray], np.ndarray]
    outlier_mask: Optional[np.ndarray] = None   # uint8 [B][Hkv][128]
    outlier_scale: float = 2.0
    step: int = 0
    steps: int = 1
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE
    meta: dict = field(default_factory=dict)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def n_max(self) -> int:
        return int(self.seq_lens.max())

    def k_per_seq(self) -> np.ndarray:
        return np.ascontiguousarray(self.k_rule(self.seq_lens), dtype=np.int32)

    def k_max(self) -> int:
        return int(self.k_per_seq().max())

    def new_rows(self):
        """K and V rows of the token each sequence appends at this step.

        Returns (tok [B], pages [B], slots [B], k_rows [B][Hkv][128], v_rows) where the
        new token tok[b] = seq_lens[b] goes to page page_table[b][tok // 16], slot tok % 16.
        """
        tok = np.ascontiguousarray(self.seq_lens, dtype=np.int32)
        if np.any(tok >= self.capacity):
            raise ValueError("workload has no planned capacity for another token")
        pages = self.page_table[np.arange(self.batch), tok // self.page_size].astype(np.int64)
        slots = (tok % self.page_size).astype(np.int64)
        lib = _load()
        kr = np.empty((self.batch, self.num_kv_heads, self.head_dim), dtype=np.uint16)
        vr = np.empty_like(kr)
        lib.synth_kv_rows(self.seed, T_K, self.batch, self.num_kv_heads, self.head_dim, _ptr(tok),
                          _ptr(self.outlier_mask), self.outlier_scale, _ptr(kr))
        lib.synth_kv_rows(self.seed, T_V, self.batch, self.num_kv_heads, self.head_dim, _ptr(tok),
                          None, 0.0, _ptr(vr))
        return tok, pages, slots, kr, vr

    def advance(self, write_host: bool = True):
        """Append one token per sequence (host copy) and draw the next step's queries."""
        tok, pages, slots, kr, vr = self.new_rows()
        if write_host:
            for b in range(self.batch):
                self.k_cache[pages[b], :, slots[b], :] = kr[b]
                self.v_cache[pages[b], :, slots[b], :] = vr[b]
        self.seq_lens = (self.seq_lens + 1).astype(np.int32)
        self.step += 1
        self.q = queries(self.seed, self.step, self.batch, self.num_q_heads, self.head_dim)
        return tok, pages, slots, kr, vr

    def logical_kv(self, which: str, b: int) -> np.ndarray:
        """Logical [Hkv][N_b][128] view of sequence b (test convenience, gathers pages)."""
        cache = self.k_cache if which == "k" else self.v_cache
        n = int(self.seq_lens[b])
        npg = (n + self.page_size - 1) // self.page_size
        pages = self.page_table[b, :npg]
        blk = cache[pages]                               # [npg][Hkv][16][128]
        blk = blk.transpose(1, 0, 2, 3).reshape(self.num_kv_heads, npg * self.page_size, self.head_dim)
        return np.ascontiguousarray(blk[:, :n, :])


def queries(seed: int, step: int, batch: int, num_q_heads: int, head_dim: int = HEAD_DIM) -> np.ndarray:
    out = np.empty((batch, num_q_heads, head_dim), dtype=np.uint16)
    _load().synth_queries(seed, step, batch, num_q_heads, head_dim, _ptr(out))
    return out


def make_page_table(layout: str, seed: int, capacity: np.ndarray, page_size: int = PAGE_SIZE,
                    initial: Optional[np.ndarray] = None):
    """Page table [B][max_pages] and pool size for a layout (see module docstring)."""
    capacity = np.asarray(capacity, dtype=np.int64)
    batch = capacity.shape[0]
    need = (capacity + page_size - 1) // page_size
    max_pages = int(max(1, need.max()))
    pt = np.zeros((batch, max_pages), dtype=np.int32)
    if layout == "contiguous":
        for b in range(batch):
            pt[b] = b * max_pages + np.arange(max_pages)
        return pt, batch * max_pages
    if layout == "shuffled":
        pool = batch * max_pages
        perm = permutation(seed, tag(T_PAGES), pool)
        return np.ascontiguousarray(perm.reshape(batch, max_pages).astype(np.int32)), pool
    if layout == "fragmented":
        pool = int(math.ceil(1.25 * int(need.sum())))
        free = list(permutation(seed, tag(T_PAGES, 1), pool))
        free.reverse()                                   # pop() takes the list's head
        init = need if initial is None else (np.asarray(initial, np.int64) + page_size - 1) // page_size
        for r in range(int(init.max())):                 # deal round-robin
            for b in range(batch):
                if r < init[b]:
                    pt[b, r] = free.pop()
        nxt = init.copy()
        while np.any(nxt < need):                        # growth pages, in step order
            for b in range(batch):
                if nxt[b] < need[b]:
                    pt[b, nxt[b]] = free.pop()
                    nxt[b] += 1
        return pt, pool
    raise ValueError(f"unknown layout {layout!r}")


def make_workload(name: str, seed: int, batch: int, num_q_heads: int, num_kv_heads: int,
                  seq_lens, k_rule, layout: str = "shuffled", growth: int = 0,
                  planted: int = 0, outlier_channels: int = 0, outlier_scale: float = 2.0,
                  steps: Optional[int] = None) -> Workload:
    """Build a workload whose cache is filled for tokens < seq_lens and has page room for
    `growth` more tokens per sequence (their values come from new_rows())."""
    lib = _load()
    seq_lens = np.ascontiguousarray(np.broadcast_to(np.asarray(seq_lens, np.int32), (batch,)))
    if np.any(seq_lens < 1):
        raise ValueError("every sequence needs at least one token")
    capacity = (seq_lens + growth).astype(np.int32)
    pt, pool = make_page_table(layout, seed, capacity, initial=seq_lens)
    shape = (pool, num_kv_heads, PAGE_SIZE, HEAD_DIM)
    k_cache = np.zeros(shape, dtype=np.uint16)
    v_cache = np.zeros(shape, dtype=np.uint16)
    lo = np.zeros(batch, dtype=np.int32)
    mask = None
    if outlier_channels:
        mask = np.zeros((batch, num_kv_heads, HEAD_DIM), dtype=np.uint8)
        for b in range(batch):
            for g in range(num_kv_heads):
                ch = permutation(seed, tag(T_CHAN, 0, b, g), HEAD_DIM)[:outlier_channels]
                mask[b, g, ch] = 1
    lib.synth_fill_kv_paged(seed, T_K, batch, num_kv_heads, HEAD_DIM, PAGE_SIZE, pt.shape[1], _ptr(pt),
                            _ptr(lo), _ptr(seq_lens), _ptr(mask), outlier_scale, _ptr(k_cache))
    lib.synth_fill_kv_paged(seed, T_V, batch, num_kv_heads, HEAD_DIM, PAGE_SIZE, pt.shape[1], _ptr(pt),
                            _ptr(lo), _ptr(seq_lens), None, 0.0, _ptr(v_cache))
    q = queries(seed, 0, batch, num_q_heads)
    wl = Workload(name=name, seed=seed, batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  seq_lens=seq_lens.copy(), capacity=capacity, page_table=pt, num_pages=pool,
                  k_cache=k_cache, v_cache=v_cache, q=q, k_rule=k_rule, outlier_mask=mask,
                  outlier_scale=outlier_scale, steps=steps if steps is not None else growth + 1)
    if planted:
        _plant_keys(wl, planted)
    wl.meta.update(layout=layout, planted=planted, outlier_channels=outlier_channels, growth=growth)
    return wl


def _plant_keys(wl: Workload, count: int):
    """Overwrite `count` seeded distinct positions of each (b, kv head) with keys along the
    unit vector of the sum of the group's step-0 queries (times sqrt(128)) plus 0.25 N(0,1)."""
    G = wl.group
    qf = bf16_to_f32(wl.q).astype(np.float64)
    positions = {}
    for b in range(wl.batch):
        n = int(wl.seq_lens[b])
        c = min(count, n)
        for g in range(wl.num_kv_heads):
            pos = np.sort(permutation(wl.seed, tag(T_POS, 0, b, g), n)[:c])
            s = qf[b, g * G:(g + 1) * G].sum(axis=0)
            u = s / np.linalg.norm(s)
            noise = normal_f64(wl.seed, tag(T_PLANT, 0, b, g), c * HEAD_DIM).reshape(c, HEAD_DIM)
            rows = round_bf16(math.sqrt(HEAD_DIM) * u[None, :] + 0.25 * noise)
            pages = wl.page_table[b, pos // PAGE_SIZE]
            wl.k_cache[pages, g, pos % PAGE_SIZE, :] = rows
            positions[(b, g)] = pos
    wl.meta["planted_positions"] = positions


# ---- the five decode configurations ----------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny: B1 Hq4/Hkv1 N4096 k82 contiguous",
    2: "llama3-8b layer: B8 Hq32/Hkv8 N32768 k655 shuffled pages, 64 planted keys",
    3: "long retrieval: B4 Hq40/Hkv8 N131072 k2621 shuffled pages, t3 outlier channels",
    4: "extreme sparsity sweep: B16 Hq32/Hkv8 N131072(+8 steps) k in N/100,N/50,N/20,N",
    5: "agentic ragged: B32 Hq64/Hkv8 N_i~U[8192,163840](+32 steps) k=ceil(N_i/50) fragmented",
}


def config(cfg: int, seed: Optional[int] = None, n: Optional[int] = None, batch: Optional[int] = None,
           ratio: Optional[int] = None, steps: Optional[int] = None) -> Workload:
    """One of the five decode configurations; n / batch / steps shrink it for tests.

    The seed defaults to the configuration number.
    """
    seed = cfg if seed is None else seed
    if cfg == 1:
        N = n or 4096
        return make_workload("C1", seed, batch or 1, 4, 1, N, k_half_up(ratio or 50), "contiguous")
    if cfg == 2:
        N = n or 32768
        return make_workload("C2", seed, batch or 8, 32, 8, N, k_half_up(ratio or 50), "shuffled",
                             planted=64)
    if cfg == 3:
        N = n or 131072
        return make_workload("C3", seed, batch or 4, 40, 8, N, k_half_up(ratio or 50), "shuffled",
                             outlier_channels=8)
    if cfg == 4:
        N = n or 131072
        st = 8 if steps is None else steps
        r = ratio or 50
        rule = k_half_up(r)
        return make_workload("C4", seed, batch or 16, 32, 8, N, rule, "shuffled", growth=st - 1, steps=st)
    if cfg == 5:
        B = batch or 32
        st = 32 if steps is None else steps
        lo, hi = 8192, 163840
        if n is not None:                      # shrunk variant: lengths in [n/20, n]
            lo, hi = max(1, n // 20), n
        draws = u64(seed, tag(T_LENS), B)
        lens = (lo + (draws % np.uint64(hi - lo + 1)).astype(np.int64)).astype(np.int32)
        return make_workload("C5", seed, B, 64, 8, lens, k_ceil(ratio or 50), "fragmented",
                             growth=st - 1, steps=st)
    raise ValueError(f"no configuration {cfg}")
