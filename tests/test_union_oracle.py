"""Union-of-routes oracle: set semantics checked by brute force and invariants."""

import numpy as np
import pytest

import oracle
import synth


def brute_union(ids, tw, E):
    # independent formulation: scan every expert id 0..E-1 in order
    L, k = ids.shape
    uniq, masks, uw = [], [], []
    for e in range(E):
        hit = ids == e
        if not hit.any():
            continue
        uniq.append(e)
        m = 0
        row = np.zeros(L, np.float32)
        for t in range(L):
            acc = np.float32(0)
            for j in range(k):
                if hit[t, j]:
                    acc = np.float32(acc + tw[t, j])
                    m |= 1 << t
            row[t] = acc
        masks.append(m)
        uw.append(row)
    return uniq, masks, np.array(uw, np.float32).reshape(len(uniq), L)


CASES = {
    "random": lambda rng: rng.integers(0, 256, size=(8, 8)),
    "all_same": lambda rng: np.full((4, 8), 17),
    "all_distinct": lambda rng: np.arange(64).reshape(8, 8)[:, ::-1],
    "dup_in_token": lambda rng: np.array([[3, 3, 5, 255], [255, 0, 0, 3]]),
    "last_id": lambda rng: np.full((3, 2), 255),
    "L32": lambda rng: rng.integers(0, 256, size=(32, 8)),
    "L1": lambda rng: rng.permutation(256)[:8].reshape(1, 8),
    "k1": lambda rng: rng.integers(0, 256, size=(7, 1)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_union_matches_brute_force(case):
    rng = np.random.default_rng(hash(case) % 2**32)
    ids = np.asarray(CASES[case](rng), np.int32)
    L, k = ids.shape
    tw = rng.uniform(0, 1, size=(L, k)).astype(np.float32)
    r = oracle.route_union(ids, tw, 256)
    uniq, masks, uw = brute_union(ids, tw, 256)
    assert r["u"] == len(set(ids.ravel().tolist())) == len(uniq)
    assert r["uniq_ids"].tolist() == uniq
    assert [int(m) for m in r["tok_mask"]] == masks
    assert np.array_equal(r["uniq_w"].view(np.uint32), uw.view(np.uint32))
    # slot -> unique index maps back to the id
    assert np.array_equal(r["uniq_ids"][r["slot_to_uniq"]], ids)
    # every token's router weight appears exactly once across the union
    assert np.allclose(r["uniq_w"].sum(0), tw.sum(1), rtol=1e-6)


def test_sorted_pairs_stable_and_offsets():
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 16, size=(12, 4)).astype(np.int32)
    r = oracle.sorted_pairs(ids, 16)
    flat = ids.ravel()
    keys = [(int(flat[p]), int(p)) for p in r["perm"]]
    assert keys == sorted(keys)
    counts = np.bincount(flat, minlength=16)
    assert np.array_equal(np.diff(r["offsets"]), counts)
    assert np.array_equal(r["perm"][r["inv"]], np.arange(flat.size))
    for e in range(16):
        seg = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert (flat[seg] == e).all()
