"""Values printed on the pages, stored under tests/golden/ with their sources."""

import os

import numpy as np

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = [s.strip() for s in line.split("=", 1)]
        vals.setdefault(key, []).append(val)
    return vals


def test_bytes_per_expert_matches_printed_size():
    import bench
    g = read_golden("bytes_per_expert.txt")
    H, I = int(g["H"][0]), int(g["I"][0])
    mb = float(g["megabytes_printed"][0])
    b = bench.expert_bytes(H, I)
    assert b == 3 * H * I // 2 + 3 * (H * I // 64) * 4
    assert round(b / 1e6, 1) == mb


def test_overlap_schedule_matches_measured_groups():
    g = read_golden("overlap_groups.txt")
    groups = [tuple(float(v) for v in s.split()) for s in g["group"]]
    sched = synth.overlap_schedule(75) * 100
    for gi, (mean, lo, hi) in enumerate(groups):
        part = sched[15 * gi:15 * (gi + 1)]
        assert abs(part.mean() - mean) < 1e-9
        assert part.min() >= lo and part.max() <= hi
    assert abs(sched.mean() - float(g["overall_mean"][0])) < 0.1
    # depth-graded: group means rise
    assert all(groups[i][0] < groups[i + 1][0] for i in range(4))


def test_overlap_chain_statistics():
    g = read_golden("overlap_groups.txt")
    target = float(g["overall_mean"][0]) / 100
    rng = np.random.default_rng(0)
    n = 4000
    shared, uniq2 = [], []
    for _ in range(n):
        ids = synth.routes_overlap_chain(2, 8, 256, target, rng)
        s = len(set(ids[0]) & set(ids[1]))
        shared.append(s / 8)
        uniq2.append(len(set(ids.ravel())))
    assert abs(np.mean(shared) - target) < 0.01
    assert abs(np.mean(uniq2) - float(g["uniques_L2"][0])) < 0.15
    # unique experts of longer chained windows, against the bank table
    by_L = dict(tuple(int(v) for v in kv.split(":")) for kv in g["uniques_by_L"][0].split())
    for L, printed in by_L.items():
        us = [len(set(synth.routes_overlap_chain(L, 8, 256, target, rng).ravel())) for _ in range(1500)]
        assert abs(np.mean(us) - printed) <= 1.5, (L, np.mean(us), printed)


def test_random_routing_overlap_is_small():
    g = read_golden("overlap_groups.txt")
    rng = np.random.default_rng(1)
    ids = [synth.routes_uniform(2, 8, 256, rng) for _ in range(3000)]
    ov = np.mean([len(set(a[0]) & set(a[1])) / 8 for a in ids]) * 100
    assert abs(ov - float(g["random_overlap_percent"][0])) < 1.0


def test_tile_schedule_worked_example():
    g = read_golden("tile_schedule.txt")
    bm = int(g["bm"][0])
    counts = [int(v) for v in g["row_counts"][0].split()]
    ids = np.concatenate([np.full(c, e) for e, c in enumerate(counts)]).astype(np.int32)
    sp = oracle.sorted_pairs(ids.reshape(-1, 1), len(counts))
    tiles = oracle.expert_tiles(sp["offsets"], bm)
    assert len(tiles) == int(g["offset_tiles"][0])
    assert oracle.naive_tile_passes(counts, bm) == int(g["naive_passes"][0])
    assert [t[2] for t in tiles] == counts
