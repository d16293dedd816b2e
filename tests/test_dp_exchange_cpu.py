"""Multi-process CPU test (gloo) of the split step's exchange: every rank receives the
bit-identical rank-order sum of the ranks' squared norms, non-finite values propagate."""
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
        from mixed_precision_zero_amd.dp import global_sumsq
        res = []
        for v in values:
            local = torch.tensor([v[rank]], dtype=torch.float64)
            res.append(global_sumsq(local).item())
        out_q.put((rank, res))
    finally:
        dist.destroy_process_group()


@pytest.mark.parametrize("world", [2, 3])
def test_global_sumsq_rank_order_and_nonfinite(world):
    # values chosen so that the summation order changes the result in the last bits
    cases = [
        [1e16, 1.0, -1e16][:world] if world == 3 else [0.1, 0.2],
        [3.0, float("inf"), 1.0][:world],
        [float("nan"), 2.0, 5.0][:world],
        [2.0 ** -1074, 1.0, 2.0 ** 60][:world],
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
        want = vals[0]
        for v in vals[1:]:
            want = want + v
        for r in range(world):
            g = got[r][i]
            if math.isnan(want):
                assert math.isnan(g)
            else:
                assert g == want and math.copysign(1, g) == math.copysign(1, want), (i, r, g, want)
        # identical bits on every rank
        assert len({repr(got[r][i]) for r in range(world)}) == 1
