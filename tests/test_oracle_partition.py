"""Pins of the oracle's shard layout: hand-derived cases and exact-cover invariants."""
import os

import numpy as np
import pytest

from oracle import oracle as O
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_cases():
    cases, cur = [], None
    with open(os.path.join(HERE, "golden", "partition_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "case":
                kv = dict(p.split("=") for p in parts[2:])
                cur = dict(name=parts[1], D=int(kv["D"]), align=int(kv["align"]),
                           numel=[int(x) for x in kv["numel"].split(",")],
                           decay=[int(x) for x in kv["decay"].split(",")], segs=[])
                cases.append(cur)
            else:
                cur["segs"].append(tuple(int(x) for x in parts[1:]))
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_partition_golden(case):
    for r in range(case["D"]):
        segs, P = O.partition(case["numel"], case["decay"], case["D"], r, case["align"])
        got = [(r, s["shard_offset"], s["numel"], s["tensor_offset"], s["tensor_id"], s["flags"])
               for s in segs]
        assert got == [s for s in case["segs"] if s[0] == r]


def check_exact_cover(numel, decay, D, align):
    total = sum(numel)
    P = None
    covered = np.zeros(len(numel) + 1, np.int64)
    for r in range(D):
        segs, P = O.partition(numel, decay, D, r, align)
        pos = 0
        for s in segs:
            assert s["shard_offset"] == pos and s["numel"] > 0
            pos += s["numel"]
            tid = s["tensor_id"]
            if tid < len(numel):
                assert s["flags"] == (1 if decay[tid] else 0)
                assert s["tensor_offset"] + s["numel"] <= numel[tid]
            else:
                assert s["flags"] == 0
            covered[tid] += s["numel"]
        assert pos == P
    assert P * D % (D * align) == 0 and P * D >= total and P * D - total < D * align
    assert list(covered[:-1]) == list(numel)
    assert covered[-1] == P * D - total
    return P


def test_partition_random_exact_cover():
    rng = np.random.default_rng(30)
    for _ in range(40):
        k = int(rng.integers(1, 12))
        numel = [int(x) for x in rng.integers(0, 50, k)]
        if sum(numel) == 0:
            numel[0] = 1
        decay = [int(x) for x in rng.integers(0, 2, k)]
        check_exact_cover(numel, decay, int(rng.integers(1, 9)), int(rng.integers(1, 9)))


def test_pythia410m_layout():
    """Rank 0 of 8 is all embedding; rank 1 holds the embedding tail, two full layers
    and the third layer up to its projection weight: 36 segments, 38,912 no-decay
    elements (2 x 13,312 + 12,288 biases and LayerNorm parameters)."""
    t = workloads.pythia410m_tensors()
    numel = [n for n, _ in t]
    decay = [int(d) for _, d in t]
    assert sum(numel) == 353_820_672
    segs0, P = O.partition(numel, decay, 8, 0, 64)
    assert P == 44_227_584 and len(segs0) == 1 and segs0[0]["tensor_id"] == 0
    segs1, _ = O.partition(numel, decay, 8, 1, 64)
    assert len(segs1) == 36
    assert sum(s["numel"] for s in segs1 if not s["flags"]) == 38_912
    for r in range(8):
        segs, _ = O.partition(numel, decay, 8, r, 64)
        w = workloads.pythia410m(r, [(s["numel"], s["flags"]) for s in segs])
        assert w.numel == P and w.name == f"pythia410m_dp8_rank{r}"
