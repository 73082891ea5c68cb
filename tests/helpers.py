"""Shared test helpers: tiny paged caches built straight from logical tensors.

The scatter into pages here is written independently of both the oracle's page
walk and the GPU kernels' addressing, so layout mistakes in either show up.
"""
from __future__ import annotations

import numpy as np

import synth


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of values that must already be exactly representable in bf16."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value not representable in bf16")
    return (bits >> 16).astype(np.uint16)


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value, returned as float64."""
    return synth.bf16_to_f32(synth.f32_to_bf16(np.asarray(x, dtype=np.float64))).astype(np.float64)


class TinyCase:
    """A paged cache + queries from logical per-sequence tensors.

    k_logical / v_logical: list over b of float arrays [Hkv][N_b][128] (bf16-exact values).
    q: float array [B][Hq][128] (bf16-exact).
    """

    def __init__(self, k_logical, v_logical, q, layout="shuffled", seed=7, extra_pages=0):
        self.batch = len(k_logical)
        self.num_kv_heads = k_logical[0].shape[0]
        self.lens = np.array([k.shape[1] for k in k_logical], dtype=np.int32)
        self.q_f = np.asarray(q, dtype=np.float64)
        self.num_q_heads = self.q_f.shape[1]
        pt, pool = synth.make_page_table(layout, seed, self.lens + extra_pages)
        self.page_table = pt
        shape = (pool, self.num_kv_heads, 16, 128)
        self.k_cache = np.zeros(shape, dtype=np.uint16)
        self.v_cache = np.zeros(shape, dtype=np.uint16)
        for b in range(self.batch):
            kb, vb = bf16_bits(k_logical[b]), bf16_bits(v_logical[b])
            for j in range(self.lens[b]):
                page = pt[b, j // 16]
                self.k_cache[page, :, j % 16, :] = kb[:, j, :]
                self.v_cache[page, :, j % 16, :] = vb[:, j, :]
        self.k_f = [np.asarray(k, dtype=np.float64) for k in k_logical]
        self.v_f = [np.asarray(v, dtype=np.float64) for v in v_logical]
        self.q = bf16_bits(self.q_f)

    @property
    def group(self):
        return self.num_q_heads // self.num_kv_heads


def random_case(rng, batch, hq, hkv, lens, layout="shuffled", integer=False, lo=-2, hi=2, seed=7):
    lens = list(np.broadcast_to(np.asarray(lens), (batch,)))
    if integer:
        draw = lambda *s: rng.integers(lo, hi + 1, size=s).astype(np.float64)
    else:
        draw = lambda *s: bf16_round(rng.standard_normal(s))
    k = [draw(hkv, int(n), 128) for n in lens]
    v = [draw(hkv, int(n), 128) for n in lens]
    q = draw(batch, hq, 128)
    return TinyCase(k, v, q, layout=layout, seed=seed)
