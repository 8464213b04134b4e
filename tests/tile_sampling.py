"""Deterministic token samples for sampled parity checks of the sorted path.

At full size the oracle checks a sample of tokens.  The sample is chosen from
the expert sort (a stable sort of the pairs by expert, cut into row tiles of
bm rows at expert boundaries) so that it holds, for each tile height the
kernels may use:
  * the first and last rows of the first and of the last tile of the experts
    with the most and with the fewest rows;
  * the last row of a final tile for every residue n_e mod bm that occurs
    (every height of a partial last tile);
  * further experts' last rows, then seeded random tokens, up to n tokens.
"""

import numpy as np

import oracle

TILE_HEIGHTS = (32, 64, 96, 128)  # 32-row MFMA blocks per tile: 1..4


def coverage_tokens(ids: np.ndarray, E: int, n: int = 64, seed: int = 0, heights=TILE_HEIGHTS) -> list:
    ids = np.asarray(ids)
    T, k = ids.shape
    s = oracle.sorted_pairs(ids, E)
    off, perm = np.asarray(s["offsets"]), np.asarray(s["perm"])
    cnt = np.diff(off)
    nz = np.flatnonzero(cnt)
    tok = lambda row: int(perm[row]) // k  # noqa: E731
    chosen = []
    for bm in heights:
        for e in (nz[np.argmax(cnt[nz])], nz[np.argmin(cnt[nz])]):
            first, last = int(off[e]), int(off[e + 1]) - 1
            last_tile = first + ((int(cnt[e]) - 1) // bm) * bm
            chosen += [tok(first), tok(min(first + bm - 1, last)), tok(last_tile), tok(last)]
        by_residue = {}
        for e in nz:
            by_residue.setdefault(int(cnt[e]) % bm, int(e))
        chosen += [tok(int(off[e + 1]) - 1) for _, e in sorted(by_residue.items())]
    out = list(dict.fromkeys(chosen))
    for e in nz:  # further final rows, ascending expert
        if len(out) >= n:
            break
        t = tok(int(off[e + 1]) - 1)
        if t not in out:
            out.append(t)
    rng = np.random.default_rng(seed)
    for t in rng.permutation(T).tolist():
        if len(out) >= n:
            break
        if t not in out:
            out.append(t)
    return sorted(out)
