"""Helpers for the GPU tests: heaps over torch memory, uploads, downloads.

Device memory and streams come from torch; every operation under test runs
through the C ABI (gemm_all_gather_amd.binding).  Nothing here computes an
expected value: those come from the oracle package.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

from gemm_all_gather_amd import binding as ag


def log(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu() -> torch.device:
    assert torch.cuda.is_available(), "a GPU test ran without a visible GPU"
    ag.lib()   # fail loudly when the library is missing
    return torch.device("cuda:0")


class TorchHeap:
    """A heap of n_ranks regions over one torch uint8 tensor."""

    def __init__(self, n_ranks: int, bytes_per_rank: int, fill16: int | None = 0x7E00):
        assert bytes_per_rank % 256 == 0
        self.n_ranks = n_ranks
        self.S = bytes_per_rank
        self.slab = torch.empty(n_ranks * bytes_per_rank, dtype=torch.uint8, device="cuda")
        if fill16 is not None:
            self.fill(fill16)
        self.heap = ag.Heap.wrap(self.slab, n_ranks, bytes_per_rank)
        self.views = {}

    def fill(self, pattern16: int) -> None:
        v = np.array([pattern16], dtype=np.uint16).view(np.int16)[0]
        self.slab.view(torch.int16).fill_(int(v))

    def fill_random(self, seed: int) -> np.ndarray:
        g = np.random.default_rng(seed)
        host = g.integers(0, 256, self.slab.numel(), dtype=np.uint8)
        self.slab.copy_(torch.from_numpy(host))
        return host

    def view(self, rank: int) -> ag.Heap:
        if rank not in self.views:
            self.views[rank] = self.heap.view(rank)
        return self.views[rank]

    def region(self, r: int) -> torch.Tensor:
        return self.slab[r * self.S:(r + 1) * self.S]

    def host(self) -> np.ndarray:
        torch.cuda.synchronize()
        return self.slab.cpu().numpy()

    def close(self) -> None:
        for v in self.views.values():
            v.destroy()
        self.views.clear()
        self.heap.destroy()


def to_device(arr: np.ndarray) -> torch.Tensor:
    """Upload a numpy array (uint16 bit patterns, float32 or bytes) as raw bytes in a device tensor."""
    a = np.ascontiguousarray(arr)
    t = torch.from_numpy(a.view(np.uint8).reshape(-1).copy()).to("cuda")
    return t


def as_typed(t: torch.Tensor, dtype: str, shape) -> torch.Tensor:
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "u16": torch.int16}[dtype]
    return t.view(tdt).reshape(shape)


def run_all_gather(th: TorchHeap, inputs_dev, W, rank_start, rank_stride, out_offset, M, N, dtype,
                   tile_m=0, tile_n=0, n_programs=0, stream=None) -> None:
    """Every group member's call, in group order, on one stream."""
    for j in range(W):
        r = rank_start + j * rank_stride
        ag.all_gather(th.view(r), W, rank_start, rank_stride, inputs_dev[j], out_offset, M, N, dtype,
                      tile_m, tile_n, n_programs, stream)
