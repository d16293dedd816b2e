"""Segment / chunk bookkeeping without a GPU: neox_zero1_plan() returns the work
decomposition create() would upload.  Chunk tables are compared bit for bit with a
brute-force construction from the rule the header states; flat tile tables are checked
by rebuilding every element's decay flag from them.  Pointers are fake integers: the
plan only compares them."""
import numpy as np
import pytest

import mixed_precision_zero_amd as Z
import workloads as W

BASE = 1 << 36                   # fake device addresses, far apart per array
STRIDE = 1 << 34


def _cfg(**over):
    return Z.neox_zero1_default_config(**over)


def flat_segments(sizes, decays, mis=(0, 0, 0, 0, 0), gap_after=None, sgd=False):
    """Segments as consecutive views of five buffers starting at BASE + k*STRIDE + mis[k]
    bytes; gap_after=i leaves a 16-byte hole in every array after segment i."""
    segs, off = [], 0
    for i, (n, d) in enumerate(zip(sizes, decays)):
        g = BASE + mis[0] + 2 * off
        h = BASE + STRIDE + mis[1] + 2 * off
        w = BASE + 2 * STRIDE + mis[2] + 4 * off
        m = BASE + 3 * STRIDE + mis[3] + 4 * off
        v = 0 if sgd else BASE + 4 * STRIDE + mis[4] + 4 * off
        segs.append(Z.neox_segment(g, h, w, m, v, n, Z.NEOX_SEG_DECAY if d else 0, i, 0))
        off += n + (8 if gap_after == i else 0)
    return segs


def separate_segments(rng, sizes, decays):
    """Each segment's arrays in their own fake allocation with a random 2- or 4-byte
    aligned start offset (so some segments align after a head, some never do)."""
    segs = []
    for i, (n, d) in enumerate(zip(sizes, decays)):
        base = BASE + i * (1 << 28)
        g = base + 2 * int(rng.integers(0, 8))
        h = base + (1 << 25) + 2 * int(rng.integers(0, 8))
        ptrs = [base + (k + 2) * (1 << 25) + 4 * int(rng.integers(0, 4)) for k in range(3)]
        segs.append(Z.neox_segment(g, h, *ptrs, n, Z.NEOX_SEG_DECAY if d else 0, i, 0))
    return segs


def expected_chunks(segs, C):
    """The chunk table by the stated rule: per segment, in order, an optional head of h < 8
    elements after which all five arrays are 16-byte aligned, then chunks of C (the head
    absent when h = 0; no vector chunks at all when no such h exists)."""
    out = []
    for k, s in enumerate(segs):
        dec = Z.NEOX_CHUNK_DECAY if s.flags & Z.NEOX_SEG_DECAY else 0
        head = next((h for h in range(8)
                     if (s.grad + 2 * h) % 16 == 0 and (s.half + 2 * h) % 16 == 0
                     and (s.master + 4 * h) % 16 == 0 and (s.exp_avg + 4 * h) % 16 == 0
                     and (not s.exp_avg_sq or (s.exp_avg_sq + 4 * h) % 16 == 0)), None)
        off = 0
        if head:
            out.append((0, k, min(head, s.numel), dec))
            off = min(head, s.numel)
        while off < s.numel:
            ln = min(C, s.numel - off)
            out.append((off, k, ln, dec | (Z.NEOX_CHUNK_VEC if head is not None else 0)))
            off += ln
    return out


def whole_span(segs):
    """One segment covering a flat partition's arrays from its first segment's start."""
    s = segs[0]
    return Z.neox_segment(s.grad, s.half, s.master, s.exp_avg, s.exp_avg_sq,
                          sum(x.numel for x in segs), s.flags, 0, 0)


def as_tuples(chunks):
    return [(c.offset, c.seg, c.len, c.flags) for c in chunks]


def decay_from_tiles(plan, words, changes):
    """Every element's decay flag rebuilt from the tile table."""
    T = plan.tile_elems
    flags = np.zeros(plan.numel, dtype=np.uint8)
    for t in range(plan.flat_tiles):
        lo, hi = t * T, min(plan.numel, (t + 1) * T)
        first, end = words[t] >> 1, words[t + 1] >> 1
        cur = words[t] & 1
        pos = lo
        for j in range(first, end):
            o = changes[j]
            assert 0 < o < T and lo + o <= hi
            flags[pos:lo + o] = cur
            pos, cur = lo + o, cur ^ 1
        flags[pos:hi] = cur
    return flags


def decay_from_segments(segs):
    return np.concatenate([np.full(s.numel, 1 if s.flags & Z.NEOX_SEG_DECAY else 0, np.uint8)
                           for s in segs])


# ---------------------------------------------------------------------------------------

def test_flat_path_selection_rules():
    sizes, decays = [5000, 3, 9000, 1], [True, False, True, False]
    plan = Z.neox_zero1_plan(_cfg(), flat_segments(sizes, decays), tables=False)[0]
    assert plan.update_path == Z.NEOX_PATH_FLAT and plan.numel == sum(sizes)
    assert plan.flat_tiles == -(-sum(sizes) // plan.tile_elems)
    for segs, cfg in [
        (flat_segments(sizes, decays), _cfg(chunked_update=1)),
        (flat_segments(sizes, decays), _cfg(chunk_elems=2048)),
        (flat_segments(sizes, decays, mis=(2, 0, 0, 0, 0)), _cfg()),     # grad not 16-aligned
        (flat_segments(sizes, decays, mis=(0, 0, 0, 0, 4)), _cfg()),     # v not 16-aligned
        (flat_segments(sizes, decays, gap_after=1), _cfg()),             # hole between segments
        (flat_segments(sizes, decays)[::-1], _cfg()),                    # out of order
    ]:
        assert Z.neox_zero1_plan(cfg, segs, tables=False)[0].update_path == Z.NEOX_PATH_CHUNKED
    # momentum SGD keeps no second moment: four contiguous arrays suffice
    sgd = flat_segments(sizes, decays, sgd=True)
    assert Z.neox_zero1_plan(_cfg(optimizer=Z.NEOX_OPT_SGD), sgd,
                             tables=False)[0].update_path == Z.NEOX_PATH_FLAT


@pytest.mark.parametrize("chunk", [0, 256, 1000, 4096])
def test_chunk_table_bruteforce(chunk):
    rng = np.random.default_rng(7 + chunk)
    for case in range(20):
        nseg = int(rng.integers(1, 12))
        sizes = [int(x) for x in rng.choice([1, 2, 7, 8, 9, 255, 256, 257, 2047, 2048, 2049,
                                             5000, 40_000, 70_001], nseg)]
        decays = [bool(x) for x in rng.integers(0, 2, nseg)]
        segs = (separate_segments(rng, sizes, decays) if case % 2 else
                flat_segments(sizes, decays, mis=tuple(int(x) for x in rng.choice([0, 4, 8], 5))
                              if case % 4 == 2 else (0,) * 5))
        cfg = _cfg(chunk_elems=chunk)
        plan, chunks, _, _ = Z.neox_zero1_plan(cfg, segs)
        C = chunk or plan.chunk_elems
        assert as_tuples(chunks) == expected_chunks(segs, C), (case, sizes)
        assert plan.update_chunks == len(chunks) and plan.numel == sum(sizes)
        # norm chunks: the smallest multiple of C that is at least the default norm length,
        # or, on a shard under 64 of those, at least numel / 64 (and at least C)
        C1 = plan.norm_chunk_elems
        target = min(32768, max(C, -(-sum(sizes) // 64)))
        assert C1 % C == 0 and C1 >= target and C1 - C < target
        # a flat partition's norm chunks cut the whole gradient, across segment bounds
        norm_segs = [whole_span(segs)] if plan.update_path == Z.NEOX_PATH_FLAT else segs
        assert plan.norm_chunks == len(expected_chunks(norm_segs, C1))


@pytest.mark.parametrize("seed", range(6))
def test_flat_tile_table_rebuilds_every_decay_flag(seed):
    rng = np.random.default_rng(100 + seed)
    nseg = int(rng.integers(1, 300))
    small = rng.integers(1, 40, nseg)
    large = rng.integers(1, 9000, nseg)
    sizes = [int(a if rng.random() < 0.6 else b) for a, b in zip(small, large)]
    decays = [bool(x) for x in rng.integers(0, 2, nseg)]
    segs = flat_segments(sizes, decays)
    plan, chunks, words, changes = Z.neox_zero1_plan(_cfg(), segs)
    assert plan.update_path == Z.NEOX_PATH_FLAT
    assert len(words) == plan.flat_tiles + 1 and len(changes) == plan.flat_changes
    assert all((a >> 1) <= (b >> 1) for a, b in zip(words, words[1:]))
    assert (words[-1] >> 1) == len(changes) and (words[-1] & 1) == 0
    assert np.array_equal(decay_from_tiles(plan, words, changes), decay_from_segments(segs))
    # the chunk table is still built (the norm pass uses its own table from the same rule)
    assert as_tuples(chunks) == expected_chunks(segs, plan.chunk_elems)


def test_plan_of_benchmark_shards():
    """The GPT-NeoX-20B per-rank shard and a Pythia-410M rank as flat partitions: tile
    count, flag changes inside tiles and chunk counts follow from the segment list."""
    t = W.pythia410m_tensors()
    psegs, _ = Z.neox_zero1_partition([n for n, _ in t], [d for _, d in t], 8, 1, 64)
    for w in (W.neox20b_shard(), W.pythia410m(1, [(s.numel, s.flags) for s in psegs])):
        sizes = [n for n, _ in w.segments]
        decays = [d for _, d in w.segments]
        segs = flat_segments(sizes, decays)
        plan, chunks, words, changes = Z.neox_zero1_plan(_cfg(), segs)
        T = plan.tile_elems
        starts = np.cumsum([0] + sizes[:-1])
        flips = [int(s) for k, s in enumerate(starts) if k and decays[k] != decays[k - 1]]
        assert plan.flat_changes == sum(1 for f in flips if f % T)
        assert plan.flat_tiles == -(-w.numel // T)
        assert plan.update_chunks == sum(-(-n // plan.chunk_elems) for n in sizes)
        assert np.array_equal(decay_from_tiles(plan, words, changes), decay_from_segments(segs))


def test_plan_errors():
    segs = flat_segments([100], [True])
    L = Z.lib()
    import ctypes as C
    arr = (Z.neox_segment * 1)(*segs)
    cfg = _cfg()
    assert L.neox_zero1_plan(C.byref(cfg), arr, 1, None, None, 0, None, 0, None, 0) == Z.NEOX_EINVAL
    out = Z.neox_zero1_plan_t()
    assert L.neox_zero1_plan(C.byref(cfg), arr, 1, C.byref(out), None, 5, None, 0, None, 0) == Z.NEOX_EINVAL
    assert L.neox_zero1_plan(None, arr, 1, C.byref(out), None, 0, None, 0, None, 0) == Z.NEOX_EINVAL
    assert L.neox_zero1_plan(C.byref(cfg), arr, 0, C.byref(out), None, 0, None, 0, None, 0) == Z.NEOX_EINVAL
    bad = _cfg(chunked_update=2)
    assert L.neox_zero1_plan(C.byref(bad), arr, 1, C.byref(out), None, 0, None, 0, None, 0) == Z.NEOX_EINVAL
    # 2^24 chunks of 256 elements: the chunk table's limit (one block per chunk)
    big = flat_segments([1 << 32], [True])
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_plan(_cfg(chunk_elems=256), big, tables=False)
    assert e.value.code == Z.NEOX_EINVAL and "chunks" in str(e.value)
    # a partial copy-out fills only what fits
    segs = flat_segments([5000, 5000], [True, False])
    plan, full, _, _ = Z.neox_zero1_plan(_cfg(chunked_update=1), segs)
    two = (Z.neox_chunk_info * 2)()
    arr2 = (Z.neox_segment * 2)(*segs)
    cfg2 = _cfg(chunked_update=1)
    assert L.neox_zero1_plan(C.byref(cfg2), arr2, 2, C.byref(out), two, 2, None, 0, None, 0) == Z.NEOX_OK
    assert as_tuples(two) == as_tuples(full[:2]) and out.update_chunks == len(full)


def test_flat_partition_beyond_the_chunk_table_limit():
    """The flat update reads no chunk table, so a flat shard of 2^35 elements (2^24 update
    chunks, more than the chunked update's grid takes) still plans as flat: 2^24 tiles,
    at most 255 norm chunks, the update deciding.  Forced onto the chunk table, the same
    shard is refused."""
    n, S = 1 << 35, 1 << 40
    segs = [Z.neox_segment(BASE, BASE + S, BASE + 2 * S, BASE + 3 * S, BASE + 4 * S, n,
                           Z.NEOX_SEG_DECAY, 0, 0)]
    plan = Z.neox_zero1_plan(_cfg(), segs, tables=False)[0]
    assert plan.update_path == Z.NEOX_PATH_FLAT and plan.flat_tiles == 1 << 24
    assert plan.update_chunks == 1 << 24 and plan.norm_chunks <= 256 and plan.update_decides == 1
    with pytest.raises(Z.NeoxError) as e:
        Z.neox_zero1_plan(_cfg(chunked_update=1), segs, tables=False)
    assert e.value.code == Z.NEOX_EINVAL and "chunks" in str(e.value)


@pytest.mark.parametrize("sizes", [[3_000_000], [2_000_000, 97, 1_500_000], [70_000_000] * 3,
                                   [1 << 31, 1 << 31], [9_000] * 200 + [5_000_000]],
                         ids=["3m", "3_segments", "210m", "4e9", "201_segments"])
def test_norm_pass_of_few_large_blocks(sizes):
    """Above 64 norm chunks of 32K elements, a flat partition's norm pass cuts its whole
    gradient into at most 256 chunks of numel / 256 elements (a multiple of the update
    chunk), whatever its segments, run as 512-thread blocks, and the update takes the
    decisions itself.  With per-segment norms the chunks must follow the segments: fewer
    than 128 segments give chunks of numel / (256 - nseg) elements, more keep 32K-element
    chunks of 256-thread blocks and a finalize; so does the chunk-table update."""
    decays = [i % 3 != 1 for i in range(len(sizes))]
    segs = flat_segments(sizes, decays)
    n, nseg = sum(sizes), len(sizes)
    plan = Z.neox_zero1_plan(_cfg(), segs, tables=False)[0]
    C = plan.chunk_elems
    few = -(-(-(-n // 256)) // C) * C
    assert plan.norm_chunk_elems == few and plan.norm_block_threads == 512
    assert plan.norm_chunks == -(-n // few) <= 256 and plan.update_decides == 1
    # per-segment norms
    plan = Z.neox_zero1_plan(_cfg(segment_norms=1), segs, tables=False)[0]
    few = -(-(-(-n // (256 - nseg))) // C) * C
    if nseg < 128 and few <= 1 << 28:
        assert plan.norm_chunk_elems == few and plan.norm_block_threads == 512
        assert plan.norm_chunks <= 256 and plan.update_decides == 1
    else:
        assert plan.norm_chunk_elems == 32768 and plan.norm_block_threads == 256
        assert plan.norm_chunks > 256 and plan.update_decides == 0
    if n < 1 << 31:      # the reference table of a 4e9-element shard is too slow to list
        assert plan.norm_chunks == len(expected_chunks(segs, plan.norm_chunk_elems))
    # a requested striding grid of at most 256 blocks decides on any layout
    plan = Z.neox_zero1_plan(_cfg(chunked_update=1, norm_blocks=200), segs, tables=False)[0]
    assert plan.update_decides == 1
    # the chunk-table update keeps the short norm chunks and the finalize
    plan = Z.neox_zero1_plan(_cfg(chunked_update=1), segs, tables=False)[0]
    assert plan.norm_chunk_elems == 32768 and plan.norm_block_threads == 256
    assert plan.update_path == Z.NEOX_PATH_CHUNKED
    assert plan.update_decides == (plan.norm_chunks <= 256)
