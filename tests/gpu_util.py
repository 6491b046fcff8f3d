"""Helpers shared by the GPU tests: upload a workload, download results."""
from __future__ import annotations

import functools

import numpy as np
import torch

import workloads

BF = torch.bfloat16


def to_dev(a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == BF:
        return torch.from_numpy(a.view(np.int16)).view(BF).cuda()
    return torch.from_numpy(a).to(dtype).cuda()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class Dev:
    """A workload's tensors on cuda:0."""

    def __init__(self, w: workloads.Workload):
        self.w = w
        self.kc = to_dev(w.key_cache, BF)
        self.vc = to_dev(w.value_cache, BF)
        self.q = to_dev(w.query, BF)
        self.bt = to_dev(w.block_tables, torch.int32)
        self.ctx = to_dev(w.context_lens, torch.int32)
        self.nk = to_dev(w.new_key, BF)
        self.nv = to_dev(w.new_value, BF)
        self.slots = to_dev(w.slot_mapping, torch.int64)


@functools.lru_cache(maxsize=None)
def workload(config: int) -> workloads.Workload:
    return workloads.make(config)


def sample_seqs(w: workloads.Workload, n: int = 6, seed: int = 0) -> list[int]:
    """Longest, shortest and a few seeded random sequences (oracle cost stays small)."""
    ctx = w.context_lens
    rng = np.random.default_rng(1000 + seed)
    pick = {int(np.argmax(ctx)), int(np.argmin(ctx))}
    extra = rng.choice(w.batch, size=min(w.batch, n), replace=False)
    for b in extra.tolist():
        if len(pick) >= n:
            break
        pick.add(int(b))
    return sorted(pick)


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)).max())
