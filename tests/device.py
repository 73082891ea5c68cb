"""Moving host workloads (synth.Workload or helpers.TinyCase) onto the GPU."""
from __future__ import annotations

import numpy as np
import torch

import sparse_attention_decode_index_amd as sdi


def bf16_tensor(bits: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def i32_tensor(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


class DeviceCase:
    """Device copies of a paged cache + queries."""

    def __init__(self, k_cache, v_cache, page_table, seq_lens, q, device="cuda"):
        self.k = bf16_tensor(k_cache, device)
        self.v = bf16_tensor(v_cache, device)
        self.pt = i32_tensor(page_table, device)
        self.sl = i32_tensor(seq_lens, device)
        self.q = bf16_tensor(q, device)
        self.kv = sdi.PagedKV(self.k, self.v, self.pt, self.sl, n_max=int(np.max(seq_lens)))

    @classmethod
    def of_workload(cls, wl, device="cuda"):
        return cls(wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.q, device)

    @classmethod
    def of_tiny(cls, case, device="cuda"):
        return cls(case.k_cache, case.v_cache, case.page_table, case.lens, case.q, device)

    def append(self, rows, q_bits, n_max):
        """Append one token per sequence with plain device copies (the cache-growth step
        of a decode loop): rows = (tok, pages, slots, k_rows, v_rows) as
        synth.Workload.new_rows returns them; then install the next step's queries."""
        tok, pages, slots, kr, vr = rows
        p = torch.from_numpy(np.asarray(pages)).to(self.k.device)
        s = torch.from_numpy(np.asarray(slots)).to(self.k.device)
        self.k[p, :, s, :] = bf16_tensor(kr, self.k.device)
        self.v[p, :, s, :] = bf16_tensor(vr, self.k.device)
        self.sl += 1
        self.q.copy_(bf16_tensor(q_bits, self.k.device))
        self.kv = sdi.PagedKV(self.k, self.v, self.pt, self.sl, n_max=int(n_max))

    def index(self, k_per_seq, k_max):
        idx = sdi.index_topk(self.kv, self.q, i32_tensor(k_per_seq), k_max)
        torch.cuda.synchronize()
        return idx.cpu().numpy()

    def attend(self, idx, k_per_seq=None, scale=sdi.DEFAULT_SCALE):
        kp = None if k_per_seq is None else i32_tensor(k_per_seq)
        out = sdi.attend(self.kv, self.q, i32_tensor(idx), kp, scale)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def dense(self, scale=sdi.DEFAULT_SCALE):
        out = sdi.dense(self.kv, self.q, scale)
        torch.cuda.synchronize()
        return out.cpu().numpy()

    def quest(self, pages_per_seq, pages_max, current_pages_only=False, summary=None):
        """(summary bf16 bits [num_pages][Hkv][2][128], token list [B][Hq][16 pages_max])."""
        summary = sdi.quest_summarize(self.kv, summary, current_pages_only)
        idx = sdi.quest_select(self.kv, self.q, summary, i32_tensor(pages_per_seq), pages_max)
        torch.cuda.synchronize()
        return summary, summary.view(torch.int16).cpu().numpy().view(np.uint16), idx.cpu().numpy()

    def label_index(self, channels, k_per_seq, k_max, current_pages_only=False, labels=None):
        """(label bits [num_pages][Hkv][16][16], indices [B][Hq][k_max])."""
        ch = i32_tensor(channels)
        labels = sdi.label_build(self.kv, ch, labels, current_pages_only)
        idx = sdi.label_index_topk(self.kv, self.q, labels, ch, i32_tensor(k_per_seq), k_max)
        torch.cuda.synchronize()
        return labels.view(torch.int16).cpu().numpy().view(np.uint16), idx.cpu().numpy()
