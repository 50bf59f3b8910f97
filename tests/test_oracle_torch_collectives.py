"""Pins the oracle's collective semantics on torch.distributed itself.

The all-gather and all-to-all results are defined as those of
torch.distributed.all_gather_into_tensor and all_to_all_single (ROCm/iris
#594, "Multi-GPU CI"; the all-to-all is the collective ROCm/iris #594,
"Compiler inspection and grouping", names next).  Three CPU processes form a
gloo group, run both collectives on seeded int32 data, and the oracle's
expected blocks must equal what each rank received.
"""

import os
import socket

import numpy as np
import pytest
import torch.multiprocessing as mp

from oracle import all_gather_expected_block, all_to_all_expected_block

W, M, N = 3, 2, 5


def _inputs():
    rng = np.random.default_rng(2024)
    return [rng.integers(-2**31, 2**31 - 1, size=(W * M, N), dtype=np.int64).astype(np.int32) for _ in range(W)]


def _rank(rank, port, q):
    import torch
    import torch.distributed as dist
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=W)
    x = torch.from_numpy(_inputs()[rank])
    a2a = torch.empty_like(x)
    dist.all_to_all_single(a2a, x)
    ag = torch.empty((W * x.shape[0], N), dtype=torch.int32)
    dist.all_gather_into_tensor(ag, x)
    q.put((rank, a2a.numpy().copy(), ag.numpy().copy()))
    dist.barrier()
    dist.destroy_process_group()


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


@pytest.mark.timeout(180)
def test_oracle_matches_torch_distributed_collectives():
    ctx = mp.get_context("spawn")
    q = ctx.Queue()
    port = _free_port()
    procs = [ctx.Process(target=_rank, args=(r, port, q)) for r in range(W)]
    for p in procs:
        p.start()
    try:
        got = {}
        for _ in range(W):
            r, a2a, ag = q.get(timeout=150)
            got[r] = (a2a, ag)
    finally:
        for p in procs:
            p.join(timeout=30)
            if p.is_alive():
                p.kill()
    ins = _inputs()
    for j in range(W):
        assert np.array_equal(got[j][0], all_to_all_expected_block(ins, j)), f"all_to_all_single, rank {j}"
        assert np.array_equal(got[j][1], all_gather_expected_block(ins)), f"all_gather_into_tensor, rank {j}"
