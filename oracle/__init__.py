"""CPU oracle for the SwitchGLU-q4 MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package.  The GPU library never calls it and shares no code
with it.

* :func:`forward_pairs`, :func:`forward_union`, :func:`output_element`,
  :func:`dequant` wrap the plain C implementation in ``moe_oracle.c`` (IEEE
  double, each (token, expert) pair evaluated on its own).
* :func:`forward_pairs_mx`, :func:`forward_union_mx`, :func:`output_element_mx`,
  :func:`dequant_mx`: the same over mxfp4 gs32 banks (FP4 E2M1 elements, one
  E8M0 power-of-two scale byte per 32 inputs).
* :func:`forward_pairs_q`, :func:`forward_union_q`, :func:`output_element_q`,
  :func:`dequant_q`: any codec of :data:`CODECS` (affine 4/8-bit with group
  32/64, mxfp4, nvfp4, mxfp8); :func:`e4m3_value` decodes one FP8 E4M3 byte.
* :func:`route_union` and :func:`sorted_pairs` are plain Python: the
  bit-exact union outputs and the expert-sorted pair order with its
  expert-aligned tile list.

Sources (web pages): the mlx discussion "Small-L fused expert gather for
fine-grained MoE decode" (implication 1 of "The data": union of routed experts,
each streamed once, applied to the positions routed to it); the page "MoE
GatherQMM small-M verify cost" (Facts: per-pair gather_qmv, the sorted grouped
path, and the expert-offset tile schedule of PR 4567 with its worked example);
the mlx issue "gather_qmm at M=1 streams 4-bit expert weights at ~half the
bandwidth of M=4" (moe_bench script: SwitchGLU order and 4-bit affine g64).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc -O2 -fopenmp (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    Lg = ctypes.c_long
    I32 = ctypes.c_int
    lib.oracle_forward_pairs_q.argtypes = [P, P, P, Lg, Lg, Lg, Lg, Lg, I32, I32, I32] + [P] * 9 + [P, P, P]
    lib.oracle_forward_pairs_q.restype = ctypes.c_int
    lib.oracle_forward_union_q.argtypes = [P, P, P, Lg, Lg, Lg, Lg, Lg, I32, I32, I32] + [P] * 9 + [P]
    lib.oracle_forward_union_q.restype = ctypes.c_int
    lib.oracle_output_element_q.argtypes = [P, P, P, Lg, Lg, Lg, Lg, Lg, I32, I32, I32] + [P] * 9 + [Lg, Lg]
    lib.oracle_output_element_q.restype = ctypes.c_double
    lib.oracle_dequant_q.argtypes = [I32, I32, I32, P, P, P, Lg, Lg, P]
    lib.oracle_dequant_q.restype = ctypes.c_int
    lib.oracle_e4m3_value.argtypes = [I32]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    _lib = lib
    return lib


def use_library(path: str):
    """Load the oracle from another build of moe_oracle.c (tests that plant
    mistakes in a copy of the source use this); returns the previous handle."""
    global _lib
    prev = _lib
    _lib = None
    global _LIB_PATH
    saved = _LIB_PATH
    _LIB_PATH = path
    try:
        _load()
    finally:
        _LIB_PATH = saved
    return prev


def restore_library(handle) -> None:
    global _lib
    _lib = handle


class OracleError(ValueError):
    pass


def _u16(a) -> np.ndarray:
    """bf16 data as a contiguous uint16 numpy array (accepts torch bf16 tensors)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            assert a.dtype == torch.bfloat16
            return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    assert a.dtype == np.uint16
    return np.ascontiguousarray(a)


def _u32(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().cpu().contiguous().numpy().view(np.uint32))
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    return np.ascontiguousarray(a.view(np.uint32) if a.dtype == np.int32 else a.astype(np.uint32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def threads() -> int:
    return int(_load().oracle_threads())


def _u8(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            assert a.dtype == torch.uint8
            return np.ascontiguousarray(a.detach().cpu().contiguous().numpy())
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(a)
    assert a.dtype == np.uint8
    return np.ascontiguousarray(a)


# --------------------------------------------------------------------------
# any codec: affine 4/8-bit (group 32/64), mxfp4, nvfp4, mxfp8
# --------------------------------------------------------------------------

#: codec name -> (format code of moe_oracle.c, bits per element, inputs per scale group)
CODECS = {
    "affine4_g64": (0, 4, 64), "affine4_g32": (0, 4, 32),
    "affine8_g64": (0, 8, 64), "affine8_g32": (0, 8, 32),
    "mxfp4": (1, 4, 32), "nvfp4": (2, 4, 16), "mxfp8": (3, 8, 32),
}


def _codec_arrays(codec: str, bank) -> List[Optional[np.ndarray]]:
    """(wg, sg, bg, wu, su, bu, wd, sd, bd) as uint32 codes, bf16 (affine) or
    uint8 scales, and bf16 biases (None for the codecs without one)."""
    fmt = CODECS[codec][0]
    ts = bank.tensors() if hasattr(bank, "tensors") else bank
    out = []
    for i, t in enumerate(ts):
        if t is None and (i % 3 != 2 or fmt == 0):
            raise OracleError(f"{codec}: array {i} of the bank is missing")
        try:
            if i % 3 == 0:
                out.append(_u32(t))
            elif i % 3 == 1:
                out.append(_u16(t) if fmt == 0 else _u8(t))
            else:
                out.append(_u16(t) if fmt == 0 else None)
        except AssertionError:
            raise OracleError(f"{codec}: array {i} of the bank has the wrong element type") from None
    return out


def _codec_shapes(codec: str, ia, ba):
    bits = CODECS[codec][1]
    L, k = ia.shape
    E, I, hw = ba[0].shape
    return L, k, E, hw * 32 // bits, I


def _p(a):
    return _ptr(a) if a is not None else None


def forward_pairs_q(codec: str, x, ids, tw, bank, want_hidden: bool = False, want_pair_out: bool = False):
    """Per-pair SwitchGLU + router-weighted combine over a bank in ``codec``.
    Returns out [L, H] float64 (and, on request, the pair hidden vectors
    [L*k, I] and pair outputs [L*k, H])."""
    fmt, bits, gs = CODECS[codec]
    xa = _u16(x)
    ia = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    wa = np.ascontiguousarray(np.asarray(tw, dtype=np.float32))
    ba = _codec_arrays(codec, bank)
    L, k, E, H, I = _codec_shapes(codec, ia, ba)
    out = np.empty((L, H), np.float64)
    hb = np.empty((L * k, I), np.float64) if want_hidden else None
    yb = np.empty((L * k, H), np.float64) if want_pair_out else None
    st = _load().oracle_forward_pairs_q(_ptr(xa), _ptr(ia), _ptr(wa), L, k, E, H, I, fmt, bits, gs,
                                        *[_p(a) for a in ba], _ptr(out), _p(hb), _p(yb))
    if st:
        raise OracleError(f"oracle_forward_pairs_q({codec}) status {st}")
    res = [out] + ([hb] if want_hidden else []) + ([yb] if want_pair_out else [])
    return res[0] if len(res) == 1 else tuple(res)


def forward_union_q(codec: str, x, ids, tw, bank) -> np.ndarray:
    """Union evaluation over a bank in ``codec``; must agree with :func:`forward_pairs_q`."""
    fmt, bits, gs = CODECS[codec]
    xa = _u16(x)
    ia = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    wa = np.ascontiguousarray(np.asarray(tw, dtype=np.float32))
    ba = _codec_arrays(codec, bank)
    L, k, E, H, I = _codec_shapes(codec, ia, ba)
    out = np.empty((L, H), np.float64)
    st = _load().oracle_forward_union_q(_ptr(xa), _ptr(ia), _ptr(wa), L, k, E, H, I, fmt, bits, gs,
                                        *[_p(a) for a in ba], _ptr(out))
    if st:
        raise OracleError(f"oracle_forward_union_q({codec}) status {st}")
    return out


def output_element_q(codec: str, x, ids, tw, bank, t: int, m: int) -> float:
    """out[t, m] alone over a bank in ``codec``."""
    fmt, bits, gs = CODECS[codec]
    xa = _u16(x)
    ia = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    wa = np.ascontiguousarray(np.asarray(tw, dtype=np.float32))
    ba = _codec_arrays(codec, bank)
    L, k, E, H, I = _codec_shapes(codec, ia, ba)
    if not (0 <= t < L and 0 <= m < H):
        raise OracleError("output_element_q: index out of range")
    return float(_load().oracle_output_element_q(_ptr(xa), _ptr(ia), _ptr(wa), L, k, E, H, I, fmt, bits, gs,
                                                 *[_p(a) for a in ba], int(t), int(m)))


def dequant_q(codec: str, W, S, B=None) -> np.ndarray:
    """Dense double copy of rows in ``codec``: W [..., N, K*bits/32] -> [..., N, K]."""
    fmt, bits, gs = CODECS[codec]
    w = _u32(W)
    s = _u16(S) if fmt == 0 else _u8(S)
    b = _u16(B) if fmt == 0 else None
    *lead, n, kw = w.shape
    K = kw * 32 // bits
    rows = int(np.prod(lead, dtype=np.int64)) * n if lead else n
    out = np.empty((rows, K), np.float64)
    st = _load().oracle_dequant_q(fmt, bits, gs, _ptr(w), _ptr(s), _p(b), rows, K, _ptr(out))
    if st:
        raise OracleError(f"oracle_dequant_q({codec}) status {st}")
    return out.reshape(*lead, n, K)


# --------------------------------------------------------------------------
# the 4-bit affine group-64 banks (nine arrays) and the six-array mxfp4 banks
# (no bias arrays): the codec entry points above
# --------------------------------------------------------------------------

def _mx_bank9(bank) -> list:
    """(wg, eg, wu, eu, wd, ed) -> the nine-array codec order with no biases."""
    ts = list(bank.tensors() if hasattr(bank, "tensors") else bank)
    return [ts[0], ts[1], None, ts[2], ts[3], None, ts[4], ts[5], None]


def _element_or_raise(v: float, what: str) -> float:
    if np.isnan(v):
        raise OracleError(f"{what}: invalid arguments")
    return v


def dequant(W, S, B) -> np.ndarray:
    """Dense double copy of packed rows: W [..., N, K/8], S/B [..., N, K/64] -> [..., N, K]."""
    return dequant_q("affine4_g64", W, S, B)


def forward_pairs(x, ids, tw, bank, want_hidden: bool = False, want_pair_out: bool = False):
    """Per-pair SwitchGLU + router-weighted combine over a 4-bit affine group-64 bank."""
    return forward_pairs_q("affine4_g64", x, ids, tw, bank, want_hidden, want_pair_out)


def forward_union(x, ids, tw, bank) -> np.ndarray:
    """Union (deduplicated) evaluation; must agree with :func:`forward_pairs`."""
    return forward_union_q("affine4_g64", x, ids, tw, bank)


def output_element(x, ids, tw, bank, t: int, m: int) -> float:
    """out[t, m] alone (per-pair evaluation of token t's k experts)."""
    return _element_or_raise(output_element_q("affine4_g64", x, ids, tw, bank, t, m), "output_element")


def dequant_mx(W, S) -> np.ndarray:
    """Dense double copy of mxfp4 rows: W [..., N, K/8], S [..., N, K/32] -> [..., N, K]."""
    return dequant_q("mxfp4", W, S)


def forward_pairs_mx(x, ids, tw, bank, want_hidden: bool = False):
    """Per-pair SwitchGLU + combine over an mxfp4 bank (wg, eg, wu, eu, wd, ed)."""
    return forward_pairs_q("mxfp4", x, ids, tw, _mx_bank9(bank), want_hidden)


def forward_union_mx(x, ids, tw, bank) -> np.ndarray:
    """Union evaluation over an mxfp4 bank; must agree with :func:`forward_pairs_mx`."""
    return forward_union_q("mxfp4", x, ids, tw, _mx_bank9(bank))


def output_element_mx(x, ids, tw, bank, t: int, m: int) -> float:
    """out[t, m] alone over an mxfp4 bank."""
    return _element_or_raise(output_element_q("mxfp4", x, ids, tw, _mx_bank9(bank), t, m), "output_element_mx")


def e4m3_value(b: int) -> float:
    """Value of one FP8 E4M3 byte."""
    return float(_load().oracle_e4m3_value(int(b)))


# --------------------------------------------------------------------------
# union of routes (bit-exact outputs)
# --------------------------------------------------------------------------

def route_union(ids, tw, E: int) -> Dict[str, np.ndarray]:
    """Distinct experts of the L*k routes and, per distinct expert, its tokens.

    Returns
      u            number of distinct experts
      uniq_ids     int32 [u]   ascending
      tok_mask     uint32 [u]  bit t set iff token t routes to the expert (L <= 32)
      uniq_w       fp32 [u, L] token t's router weights for the expert, summed
                   over its slots in ascending slot order in fp32; 0 if none
      slot_to_uniq int32 [L, k] position of ids[t, j] in uniq_ids
    Raises OracleError for ids outside [0, E).
    """
    ids = np.asarray(ids, dtype=np.int64)
    tw = np.asarray(tw, dtype=np.float32)
    L, k = ids.shape
    if ((ids < 0) | (ids >= E)).any():
        raise OracleError("expert id outside [0, E)")
    uniq = sorted(set(int(v) for v in ids.ravel()))
    pos = {e: i for i, e in enumerate(uniq)}
    u = len(uniq)
    mask = np.zeros(u, np.uint32)
    uw = np.zeros((u, L), np.float32)
    s2u = np.zeros((L, k), np.int32)
    for t in range(L):
        for j in range(k):
            i = pos[int(ids[t, j])]
            s2u[t, j] = i
            if t < 32:
                mask[i] |= np.uint32(1 << t)
            uw[i, t] = np.float32(uw[i, t] + tw[t, j])
    return {"u": u, "uniq_ids": np.array(uniq, np.int32), "tok_mask": mask,
            "uniq_w": uw, "slot_to_uniq": s2u}


# --------------------------------------------------------------------------
# expert-sorted pair order and tile schedule
# --------------------------------------------------------------------------

def sorted_pairs(ids, E: int) -> Dict[str, np.ndarray]:
    """Stable sort of the flat pair index p = t * k + j by (ids[p], p).

    Returns offsets int32 [E+1] (prefix sums of per-expert pair counts),
    perm int32 [P] (sorted position -> pair) and inv int32 [P] (pair -> sorted
    position).
    """
    ids = np.asarray(ids, dtype=np.int64).ravel()
    if ((ids < 0) | (ids >= E)).any():
        raise OracleError("expert id outside [0, E)")
    P = ids.size
    perm = sorted(range(P), key=lambda p: (int(ids[p]), p))
    counts = np.zeros(E, np.int64)
    for p in range(P):
        counts[ids[p]] += 1
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.array(perm, np.int32)
    inv = np.empty(P, np.int32)
    inv[perm] = np.arange(P, dtype=np.int32)
    return {"offsets": offsets, "perm": perm, "inv": inv}


def expert_tiles(offsets, bm: int) -> List[Tuple[int, int, int]]:
    """Row tiles that never straddle experts: ceil(n_e / bm) tiles of expert e.

    Each tile is (expert, first sorted row, rows).  This is the schedule the
    pages describe for PR 4567, built from the expert offsets.
    """
    tiles = []
    offsets = np.asarray(offsets)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        r = a
        while r < b:
            n = min(bm, b - r)
            tiles.append((e, r, n))
            r += n
    return tiles


def naive_tile_passes(row_counts, bm: int) -> int:
    """Expert passes when tiles of bm rows are cut from the sorted rows regardless
    of expert boundaries (each tile does one pass per expert it touches)."""
    bounds = np.concatenate([[0], np.cumsum(row_counts)])
    total = int(bounds[-1])
    passes = 0
    for r0 in range(0, total, bm):
        r1 = min(total, r0 + bm)
        for e in range(len(row_counts)):
            if bounds[e] < r1 and bounds[e + 1] > r0:
                passes += 1
    return passes
