"""Multi-process CPU test (gloo) of the split step's exchange: every rank receives every
rank's squared norm, in rank order, bit for bit (non-finite values included); the
library's finalize then adds them in one fixed order on every rank (GPU tests)."""
import math
import os
import socket

import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _worker(rank, world, port, values, out_q):
    os.environ["MASTER_ADDR"] = "127.0.0.1"
    os.environ["MASTER_PORT"] = str(port)
    dist.init_process_group("gloo", rank=rank, world_size=world)
    try:
        from mixed_precision_zero_amd.dp import gather_sumsq
        res = []
        for v in values:
            local = torch.tensor([v[rank]], dtype=torch.float64)
            g = gather_sumsq(local)
            assert g.dtype == torch.float64 and g.is_contiguous() and g.numel() == world
            res.append([float(x) for x in g.tolist()])
        out_q.put((rank, res))
    finally:
        dist.destroy_process_group()


@pytest.mark.parametrize("world", [2, 3])
def test_gather_sumsq_rank_order_bit_for_bit(world):
    cases = [
        [1e16, 1.0, -1e16][:world],
        [3.0, float("inf"), 1.0][:world],
        [float("nan"), 2.0, 5.0][:world],
        [2.0 ** -1074, -0.0, 2.0 ** 60][:world],
    ]
    ctx = mp.get_context("spawn")
    q = ctx.Queue()
    port = _free_port()
    procs = [ctx.Process(target=_worker, args=(r, world, port, cases, q)) for r in range(world)]
    for p in procs:
        p.start()
    got = dict(q.get(timeout=120) for _ in range(world))
    for p in procs:
        p.join(timeout=60)
        assert p.exitcode == 0
    for i, vals in enumerate(cases):
        for r in range(world):
            g = got[r][i]
            assert len(g) == world
            for a, b in zip(g, vals):
                if math.isnan(b):
                    assert math.isnan(a)
                else:
                    assert a == b and math.copysign(1, a) == math.copysign(1, b), (i, r, g, vals)
