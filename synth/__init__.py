"""Seeded synthetic inputs for the SwitchGLU-q4 MoE layer.

This module only draws random inputs and encodes them into the packed
4-bit storage format; it holds none of the layer's arithmetic (no dequant,
no matmul, no activation, no combine).  Both the CPU oracle's tests and the
GPU path's tests and benchmark take their inputs from here.

Sources for the recipes (the pages are the mlx discussion "Small-L fused
expert gather for fine-grained MoE decode" (p1), the mlx issue "gather_qmm at
M=1 streams 4-bit expert weights at ~half the bandwidth of M=4" (p3) and the
splash PR "Apple7/8 MoE gate and up in one decode pass" (p4)):

* weights: random normal, cast to bf16, then quantized affine 4-bit with a
  group of 64 (p3, "Numbers" section and its moe_bench script);
* expert ids: drawn per token without replacement (p3 script);
* adjacent-token overlap: per-depth-group means, minima and maxima of the
  measured overlap table (p1, "The data" section);
* pooled routes: 8-32 rows whose experts come from a shared pool (p4, results
  table of the expert-kernel benchmark).

Storage format (the reading taken here; the pages give shapes only):
element ``c`` of an output row sits in nibble ``c % 8`` of 32-bit word
``c // 8``, lowest nibble first; a (scale, bias) pair of bf16 values covers
each run of 64 consecutive elements along the input dimension.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

GROUP = 64
BITS = 4


# --------------------------------------------------------------------------
# seeds
# --------------------------------------------------------------------------

def sub_seed(*parts) -> int:
    """Deterministic 63-bit seed from a tuple of labels (stable across runs)."""
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def torch_gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(*parts))
    return g


def np_rng(*parts) -> np.random.Generator:
    return np.random.default_rng(sub_seed(*parts))


# --------------------------------------------------------------------------
# 4-bit affine encoding (input preparation only)
# --------------------------------------------------------------------------

def quantize_q4_g64(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Encode bf16 rows ``w[..., N, K]`` as packed 4-bit codes plus bf16 scale/bias.

    Per group of 64: lo = min, hi = max, scale = bf16((hi - lo) / 15),
    bias = bf16(lo), code = clamp(round_half_even((w - bias) / scale), 0, 15)
    (code 0 when the scale is 0).  The pages call mlx's quantizer without
    printing its formula; this min/max recipe is the plain affine one and only
    produces test data -- both compared paths consume the same bytes.

    Returns (packed int32 [..., N, K/8] holding uint32 bit patterns,
    scale bf16 [..., N, K/64], bias bf16 [..., N, K/64]).
    """
    assert w.dtype == torch.bfloat16
    *lead, n, k = w.shape
    assert k % GROUP == 0
    wf = w.float().reshape(*lead, n, k // GROUP, GROUP)
    lo = wf.amin(-1)
    hi = wf.amax(-1)
    s = ((hi - lo) / 15.0).to(torch.bfloat16)
    b = lo.to(torch.bfloat16)
    sf = s.float().unsqueeze(-1)
    bf = b.float().unsqueeze(-1)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.round((wf - bf) / safe)
    q = torch.where(sf > 0, q, torch.zeros_like(q)).clamp_(0, 15).to(torch.int64)
    packed = pack_codes(q.reshape(*lead, n, k))
    return packed, s, b


def pack_codes(q: torch.Tensor) -> torch.Tensor:
    """Pack integer codes ``q[..., K]`` (0..15) into int32 words, lowest nibble first."""
    *lead, k = q.shape
    assert k % 8 == 0
    q = q.to(torch.int64).reshape(*lead, k // 8, 8)
    shifts = torch.arange(0, 32, 4, device=q.device, dtype=torch.int64)
    words = (q << shifts).sum(-1)
    words = torch.where(words >= (1 << 31), words - (1 << 32), words)
    return words.to(torch.int32)


# --------------------------------------------------------------------------
# mxfp4 gs32 encoding (input preparation only)
# --------------------------------------------------------------------------

MX_GROUP = 32
# magnitudes of the FP4 E2M1 codes 0..7 (codes 8..15 are their negatives)
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4_g32(w: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    """Encode bf16 rows ``w[..., N, K]`` as packed FP4 E2M1 codes plus one
    E8M0 scale byte per 32 inputs (the OCP MX recipe): the block exponent is
    floor(log2(max|w|)) - 2 (E2M1's largest exponent), each element divided by
    2^exponent goes to the nearest E2M1 magnitude (ties to the even code,
    saturating at 6), and the sign becomes bit 3.  Only produces test data.

    Returns (packed int32 [..., N, K/8], scale uint8 [..., N, K/32]).
    """
    assert w.dtype == torch.bfloat16
    *lead, n, k = w.shape
    assert k % MX_GROUP == 0
    wf = w.float().reshape(*lead, n, k // MX_GROUP, MX_GROUP)
    amax = wf.abs().amax(-1)
    expo = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                       torch.full_like(amax, -127.0))
    e = (expo + 127).clamp(0, 254)
    scaled = wf / torch.exp2(e - 127).unsqueeze(-1)
    grid = torch.tensor(E2M1_MAGNITUDES, dtype=torch.float32, device=w.device)
    dist = (scaled.abs().unsqueeze(-1) - grid).abs()
    dist = dist + 1e-6 * (torch.arange(8, device=w.device) % 2)  # ties to the even code
    mag = dist.argmin(-1)
    code = mag + 8 * (scaled < 0).to(mag.dtype)
    packed = pack_codes(code.reshape(*lead, n, k))
    return packed, e.to(torch.uint8)


# --------------------------------------------------------------------------
# further codecs (input preparation only): affine 4/8-bit with group 32/64,
# nvfp4 (E2M1 x E4M3 per 16), mxfp8 (E4M3 x E8M0 per 32)
# --------------------------------------------------------------------------

def e4m3_grid(device="cpu") -> torch.Tensor:
    """Magnitudes of the FP8 E4M3 codes 0..126 (OCP: exponent bias 7, 3
    mantissa bits, exponent 0 subnormal, code 127 NaN), increasing."""
    vals = []
    for c in range(127):
        e, m = c >> 3, c & 7
        vals.append(m / 8.0 * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return torch.tensor(vals, dtype=torch.float64, device=device)


def encode_e4m3(v: torch.Tensor) -> torch.Tensor:
    """Nearest E4M3 code of each value (ties to the even code, saturating at
    448); uint8."""
    grid = e4m3_grid(v.device)
    a = v.double().abs().clamp(max=448.0)
    hi = torch.searchsorted(grid, a).clamp(max=126)
    lo = (hi - 1).clamp(min=0)
    dlo = (a - grid[lo]).abs()
    dhi = (grid[hi] - a).abs()
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo)
    return (code + 128 * (v < 0).to(code.dtype)).to(torch.uint8)


def decode_e4m3(code: torch.Tensor) -> torch.Tensor:
    """Values of E4M3 codes (float64), for the encoders' own use."""
    grid = torch.cat([e4m3_grid(code.device), torch.tensor([float("nan")], dtype=torch.float64,
                                                          device=code.device)])
    c = code.to(torch.int64)
    mag = grid[c & 127]
    return torch.where((c & 128) != 0, -mag, mag)


def pack_codes8(q: torch.Tensor) -> torch.Tensor:
    """Pack integer codes ``q[..., K]`` (0..255) into int32 words, lowest byte first."""
    *lead, k = q.shape
    assert k % 4 == 0
    q = q.to(torch.int64).reshape(*lead, k // 4, 4)
    shifts = torch.arange(0, 32, 8, device=q.device, dtype=torch.int64)
    words = (q << shifts).sum(-1)
    words = torch.where(words >= (1 << 31), words - (1 << 32), words)
    return words.to(torch.int32)


def quantize_affine(w: torch.Tensor, bits: int, gs: int):
    """Affine encoding with ``bits`` (4 or 8) and group ``gs``: the recipe of
    :func:`quantize_q4_g64` with 2^bits - 1 levels."""
    assert w.dtype == torch.bfloat16 and bits in (4, 8)
    *lead, n, k = w.shape
    assert k % gs == 0
    levels = float((1 << bits) - 1)
    wf = w.float().reshape(*lead, n, k // gs, gs)
    lo = wf.amin(-1)
    hi = wf.amax(-1)
    s = ((hi - lo) / levels).to(torch.bfloat16)
    b = lo.to(torch.bfloat16)
    sf = s.float().unsqueeze(-1)
    bf = b.float().unsqueeze(-1)
    safe = torch.where(sf > 0, sf, torch.ones_like(sf))
    q = torch.round((wf - bf) / safe)
    q = torch.where(sf > 0, q, torch.zeros_like(q)).clamp_(0, levels).to(torch.int64)
    q = q.reshape(*lead, n, k)
    return (pack_codes8(q) if bits == 8 else pack_codes(q)), s, b


def _nearest_e2m1(scaled: torch.Tensor) -> torch.Tensor:
    grid = torch.tensor(E2M1_MAGNITUDES, dtype=torch.float32, device=scaled.device)
    dist = (scaled.abs().unsqueeze(-1) - grid).abs()
    dist = dist + 1e-6 * (torch.arange(8, device=scaled.device) % 2)  # ties to the even code
    mag = dist.argmin(-1)
    return mag + 8 * (scaled < 0).to(mag.dtype)


def quantize_nvfp4_g16(w: torch.Tensor):
    """nvfp4: per 16 inputs an E4M3 scale nearest to max|w| / 6, then each
    element divided by that scale goes to the nearest E2M1 value (ties to the
    even code, saturating at 6).  Returns (packed int32 [..., N, K/8], scale
    uint8 [..., N, K/16], None)."""
    assert w.dtype == torch.bfloat16
    *lead, n, k = w.shape
    assert k % 16 == 0
    wf = w.float().reshape(*lead, n, k // 16, 16)
    sc = encode_e4m3(wf.abs().amax(-1).double() / 6.0)
    sv = decode_e4m3(sc).float().unsqueeze(-1)
    scaled = torch.where(sv > 0, wf / torch.where(sv > 0, sv, torch.ones_like(sv)), torch.zeros_like(wf))
    code = _nearest_e2m1(scaled)
    return pack_codes(code.reshape(*lead, n, k)), sc, None


def quantize_mxfp8_g32(w: torch.Tensor):
    """mxfp8 (OCP MX): block exponent floor(log2(max|w|)) - 8 (E4M3's largest
    exponent), elements divided by 2^exponent go to the nearest E4M3 value
    (ties to even, saturating at 448).  Returns (packed int32 [..., N, K/4],
    scale uint8 [..., N, K/32], None)."""
    assert w.dtype == torch.bfloat16
    *lead, n, k = w.shape
    assert k % 32 == 0
    wf = w.float().reshape(*lead, n, k // 32, 32)
    amax = wf.abs().amax(-1)
    expo = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 8,
                       torch.full_like(amax, -127.0))
    e = (expo + 127).clamp(0, 254)
    scaled = wf / torch.exp2(e - 127).unsqueeze(-1)
    code = encode_e4m3(scaled)
    return pack_codes8(code.reshape(*lead, n, k)), e.to(torch.uint8), None


#: codec name -> (bits per element, inputs per scale group, has bias)
CODECS = {
    "affine4_g64": (4, 64, True), "affine4_g32": (4, 32, True),
    "affine8_g64": (8, 64, True), "affine8_g32": (8, 32, True),
    "mxfp4": (4, 32, False), "nvfp4": (4, 16, False), "mxfp8": (8, 32, False),
}


def quantize_codec(codec: str, w: torch.Tensor):
    """(packed codes, scales, biases or None) of bf16 rows in ``codec``."""
    bits, gs, _ = CODECS[codec]
    if codec.startswith("affine"):
        return quantize_affine(w, bits, gs)
    if codec == "mxfp4":
        p, sc = quantize_mxfp4_g32(w)
        return p, sc, None
    if codec == "nvfp4":
        return quantize_nvfp4_g16(w)
    if codec == "mxfp8":
        return quantize_mxfp8_g32(w)
    raise ValueError(codec)


@dataclasses.dataclass
class BankQ:
    """One MoE layer's expert bank in any codec of :data:`CODECS` (biases None
    for the codecs without one)."""
    codec: str
    wg: torch.Tensor
    sg: torch.Tensor
    bg: Optional[torch.Tensor]
    wu: torch.Tensor
    su: torch.Tensor
    bu: Optional[torch.Tensor]
    wd: torch.Tensor
    sd: torch.Tensor
    bd: Optional[torch.Tensor]

    @property
    def E(self) -> int:
        return self.wg.shape[0]

    def tensors(self):
        return (self.wg, self.sg, self.bg, self.wu, self.su, self.bu, self.wd, self.sd, self.bd)

    def to(self, device) -> "BankQ":
        return BankQ(self.codec, *[None if t is None else t.to(device) for t in self.tensors()])

    def select(self, experts) -> "BankQ":
        idx = torch.as_tensor(experts, dtype=torch.long, device=self.wg.device)
        return BankQ(self.codec, *[None if t is None else t.index_select(0, idx) for t in self.tensors()])


def gen_matrix_q(codec: str, E: int, N: int, K: int, seed_parts, device="cpu", experts_per_chunk: int = 8):
    """E random N(0,1) matrices [N, K] -> bf16 -> ``codec``, generated in chunks."""
    parts = []
    gen = torch_gen(device, *seed_parts)
    for e0 in range(0, E, experts_per_chunk):
        e1 = min(E, e0 + experts_per_chunk)
        w = torch.randn((e1 - e0, N, K), generator=gen, device=device, dtype=torch.float32)
        parts.append(quantize_codec(codec, w.to(torch.bfloat16)))
        del w
    cat = lambda i: None if parts[0][i] is None else torch.cat([p[i] for p in parts])  # noqa: E731
    return cat(0), cat(1), cat(2)


def gen_bank_q(codec: str, E: int, H: int, I: int, seed_parts, device="cpu", experts_per_chunk: int = 8) -> BankQ:
    g = gen_matrix_q(codec, E, I, H, (*seed_parts, codec, "gate"), device, experts_per_chunk)
    u = gen_matrix_q(codec, E, I, H, (*seed_parts, codec, "up"), device, experts_per_chunk)
    d = gen_matrix_q(codec, E, H, I, (*seed_parts, codec, "down"), device, experts_per_chunk)
    return BankQ(codec, *g, *u, *d)


# --------------------------------------------------------------------------
# weights, activations, routes
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Bank:
    """One MoE layer's expert bank in packed form (all tensors on one device)."""
    wg: torch.Tensor  # int32 [E, I, H/8]
    sg: torch.Tensor  # bf16  [E, I, H/64]
    bg: torch.Tensor
    wu: torch.Tensor  # int32 [E, I, H/8]
    su: torch.Tensor
    bu: torch.Tensor
    wd: torch.Tensor  # int32 [E, H, I/8]
    sd: torch.Tensor  # bf16  [E, H, I/64]
    bd: torch.Tensor

    @property
    def E(self) -> int:
        return self.wg.shape[0]

    def tensors(self):
        return (self.wg, self.sg, self.bg, self.wu, self.su, self.bu, self.wd, self.sd, self.bd)

    def to(self, device) -> "Bank":
        return Bank(*[t.to(device) for t in self.tensors()])

    def select(self, experts) -> "Bank":
        idx = torch.as_tensor(experts, dtype=torch.long, device=self.wg.device)
        return Bank(*[t.index_select(0, idx) for t in self.tensors()])


def gen_matrix_q4(E: int, N: int, K: int, seed_parts, device="cpu", experts_per_chunk: int = 8):
    """E random N(0,1) matrices [N, K] -> bf16 -> 4-bit affine g64, generated in chunks."""
    packed = torch.empty((E, N, K // 8), dtype=torch.int32, device=device)
    scale = torch.empty((E, N, K // GROUP), dtype=torch.bfloat16, device=device)
    bias = torch.empty_like(scale)
    gen = torch_gen(device, *seed_parts)
    for e0 in range(0, E, experts_per_chunk):
        e1 = min(E, e0 + experts_per_chunk)
        w = torch.randn((e1 - e0, N, K), generator=gen, device=device, dtype=torch.float32)
        p, s, b = quantize_q4_g64(w.to(torch.bfloat16))
        packed[e0:e1], scale[e0:e1], bias[e0:e1] = p, s, b
        del w, p, s, b
    return packed, scale, bias


def gen_bank(E: int, H: int, I: int, seed_parts, device="cpu", experts_per_chunk: int = 8) -> Bank:
    g = gen_matrix_q4(E, I, H, (*seed_parts, "gate"), device, experts_per_chunk)
    u = gen_matrix_q4(E, I, H, (*seed_parts, "up"), device, experts_per_chunk)
    d = gen_matrix_q4(E, H, I, (*seed_parts, "down"), device, experts_per_chunk)
    return Bank(*g, *u, *d)


@dataclasses.dataclass
class BankMX:
    """One MoE layer's expert bank in mxfp4 gs32 form."""
    wg: torch.Tensor  # int32 [E, I, H/8]
    sg: torch.Tensor  # uint8 [E, I, H/32]
    wu: torch.Tensor
    su: torch.Tensor
    wd: torch.Tensor  # int32 [E, H, I/8]
    sd: torch.Tensor  # uint8 [E, H, I/32]

    @property
    def E(self) -> int:
        return self.wg.shape[0]

    def tensors(self):
        return (self.wg, self.sg, self.wu, self.su, self.wd, self.sd)

    def to(self, device) -> "BankMX":
        return BankMX(*[t.to(device) for t in self.tensors()])

    def select(self, experts) -> "BankMX":
        idx = torch.as_tensor(experts, dtype=torch.long, device=self.wg.device)
        return BankMX(*[t.index_select(0, idx) for t in self.tensors()])


def gen_matrix_mx(E: int, N: int, K: int, seed_parts, device="cpu", experts_per_chunk: int = 8):
    """E random N(0,1) matrices [N, K] -> bf16 -> mxfp4 gs32, generated in chunks."""
    packed = torch.empty((E, N, K // 8), dtype=torch.int32, device=device)
    scale = torch.empty((E, N, K // MX_GROUP), dtype=torch.uint8, device=device)
    gen = torch_gen(device, *seed_parts)
    for e0 in range(0, E, experts_per_chunk):
        e1 = min(E, e0 + experts_per_chunk)
        w = torch.randn((e1 - e0, N, K), generator=gen, device=device, dtype=torch.float32)
        p, sc = quantize_mxfp4_g32(w.to(torch.bfloat16))
        packed[e0:e1], scale[e0:e1] = p, sc
        del w, p, sc
    return packed, scale


def gen_bank_mx(E: int, H: int, I: int, seed_parts, device="cpu", experts_per_chunk: int = 8) -> BankMX:
    g = gen_matrix_mx(E, I, H, (*seed_parts, "gate"), device, experts_per_chunk)
    u = gen_matrix_mx(E, I, H, (*seed_parts, "up"), device, experts_per_chunk)
    d = gen_matrix_mx(E, H, I, (*seed_parts, "down"), device, experts_per_chunk)
    return BankMX(*g, *u, *d)


def gen_x(L: int, H: int, seed_parts, device="cpu") -> torch.Tensor:
    gen = torch_gen(device, *seed_parts, "x")
    return torch.randn((L, H), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def router_weights(L: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """Softmax over the k drawn experts' N(0,1) logits, per token (fp32)."""
    logits = rng.standard_normal((L, k))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def routes_uniform(L: int, k: int, E: int, rng: np.random.Generator) -> np.ndarray:
    """Independent top-k per token: k distinct experts uniform from E."""
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(L)]).astype(np.int32) \
        if L > 0 else np.zeros((0, k), np.int32)


def routes_overlap_chain(L: int, k: int, E: int, overlap: float, rng: np.random.Generator) -> np.ndarray:
    """Adjacent-token overlap chain.

    Token 0 takes k distinct experts uniformly.  Token t+1 keeps
    c ~ Binomial(k, overlap) experts of token t's set and draws k - c fresh
    ones from the experts token t did not use; slot order is shuffled.  The
    expected shared fraction of adjacent tokens is ``overlap`` and the expected
    unique count of a pair is k * (2 - overlap): 13.3 at the 34.1 % mean that
    the small-L discussion reports for GLM-5.2 router traces.
    """
    out = np.zeros((L, k), np.int32)
    if L == 0:
        return out
    prev = rng.choice(E, size=k, replace=False)
    out[0] = prev
    for t in range(1, L):
        c = int(rng.binomial(k, overlap))
        shared = rng.choice(prev, size=c, replace=False)
        rest = np.setdiff1d(np.arange(E), prev, assume_unique=False)
        fresh = rng.choice(rest, size=k - c, replace=False)
        cur = np.concatenate([shared, fresh])
        rng.shuffle(cur)
        out[t] = cur
        prev = cur
    return out


def routes_pooled(L: int, k: int, E: int, pool: int, rng: np.random.Generator) -> np.ndarray:
    """Pooled routes: one pool of ``pool`` experts per layer, each token takes k of it."""
    p = rng.choice(E, size=pool, replace=False)
    return np.stack([rng.choice(p, size=k, replace=False) for _ in range(L)]).astype(np.int32)


# Per-depth-group overlap statistics measured on router traces (p1, "The data"
# section): 5 groups of 15 MoE layers, (mean, min, max) in percent.
OVERLAP_GROUPS = [
    (21.1, 3.8, 35.3),
    (32.2, 23.6, 43.1),
    (32.5, 26.4, 38.3),
    (39.8, 31.8, 42.8),
    (44.7, 37.1, 52.1),
]


def overlap_schedule(n_layers: int = 75) -> np.ndarray:
    """Per-layer adjacent-token overlap fractions, rising with depth.

    The layers split into 5 equal depth groups.  Inside a group the values
    are evenly spaced and symmetric about the group's measured mean, with the
    half-width min(mean - min, max - mean), so every value stays within the
    group's measured range and each group's mean is exact; the overall mean
    is 34.06 %.
    """
    vals = []
    ng = len(OVERLAP_GROUPS)
    per = [n_layers // ng + (1 if g < n_layers % ng else 0) for g in range(ng)]
    for (mean, lo, hi), n in zip(OVERLAP_GROUPS, per):
        d = min(mean - lo, hi - mean)
        for i in range(n):
            frac = (2.0 * (i + 0.5) / n - 1.0) if n > 1 else 0.0
            vals.append((mean + d * frac) / 100.0)
    return np.array(vals)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int
    k: int
    H: int
    I: int
    Ls: Tuple[int, ...]
    routing: str          # "uniform" | "overlap" | "pooled"
    n_layers: int
    pool: int = 16


WORKLOADS: Dict[str, Workload] = {
    # Tiny SwitchGLU-q4: E=8, top-2, hidden 256, inter 128, L=2, seed 0.
    "tiny": Workload("tiny_E8_k2_H256_I128", 8, 2, 256, 128, (2,), "uniform", 1),
    # GLM-5.3-Flash-shaped layer (p3's shape): E=288 top-8 H=4096 I=2048.
    "flash": Workload("glm53flash_E288_k8_H4096_I2048", 288, 8, 4096, 2048, (1, 4), "uniform", 42),
    # GLM-5.2-style verify windows with the measured depth-graded overlap (p1).
    "verify": Workload("glm52verify_E256_k8_H6144_I2048", 256, 8, 6144, 2048, (1, 2, 3, 4, 8), "overlap", 75),
    # Small-expert verify rows, random and pooled routes (p4's 35B-A3B shape).
    "small": Workload("smallexpert_E256_k8_H2048_I512", 256, 8, 2048, 512, (8, 16, 32), "uniform", 16),
    "small_pooled": Workload("smallexpert_pooled_E256_k8_H2048_I512", 256, 8, 2048, 512, (8, 16, 32), "pooled", 16),
    # Prefill sorted path: T=512 / 2048 tokens.
    "prefill": Workload("prefill_E256_k8_H4096_I2048", 256, 8, 4096, 2048, (512, 2048), "uniform", 4),
}


@dataclasses.dataclass
class LayerInput:
    """Inputs of one MoE layer call (host numpy for routes, torch for the rest)."""
    x: torch.Tensor            # bf16 [L, H]
    ids: np.ndarray            # int32 [L, k] (indices into ``bank``)
    weights: np.ndarray        # fp32 [L, k]
    bank: Bank
    global_ids: np.ndarray     # int32 [L, k] ids in the full E-expert numbering


def layer_routes(w: Workload, L: int, layer: int, seed: int) -> Tuple[np.ndarray, np.ndarray]:
    rng = np_rng(seed, w.name, L, layer, "routes")
    if w.routing == "uniform":
        ids = routes_uniform(L, w.k, w.E, rng)
    elif w.routing == "overlap":
        o = overlap_schedule(w.n_layers)[layer % w.n_layers]
        ids = routes_overlap_chain(L, w.k, w.E, float(o), rng)
    elif w.routing == "pooled":
        ids = routes_pooled(L, w.k, w.E, w.pool, rng)
    else:
        raise ValueError(w.routing)
    tw = router_weights(L, w.k, np_rng(seed, w.name, L, layer, "router"))
    return ids, tw


def compact_ids(ids: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Order-preserving remap of the used expert ids to 0..E_used-1.

    Returns (used global ids ascending, remapped ids).  A compact bank holds
    only the experts a layer's routes touch, which keeps unique counts, masks,
    overlap and bytes exactly as with the full bank.
    """
    used = np.unique(ids)
    remap = np.searchsorted(used, ids).astype(np.int32)
    return used.astype(np.int32), remap


def make_layer(w: Workload, L: int, layer: int, seed: int = 0, device="cpu", compact: bool = True,
               experts_per_chunk: int = 8) -> LayerInput:
    """Generate one layer's inputs.  With ``compact`` only the used experts are materialised.

    Expert e of layer ``layer`` always gets the same weights whether the bank
    is compact or full (each expert's matrices come from their own seed).
    """
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    if compact:
        used, remap = compact_ids(ids)
    else:
        used, remap = np.arange(w.E, dtype=np.int32), ids
    bank = gen_bank_experts(w, used, layer, seed, device, experts_per_chunk)
    return LayerInput(x=x, ids=remap, weights=tw, bank=bank, global_ids=ids)


def gen_bank_experts(w: Workload, experts, layer: int, seed: int, device="cpu", experts_per_chunk: int = 8) -> Bank:
    """Bank holding the listed experts of a layer; expert e's bytes depend only on (seed, layer, e)."""
    experts = [int(e) for e in experts]
    n = len(experts)
    H, I = w.H, w.I
    wg = torch.empty((n, I, H // 8), dtype=torch.int32, device=device)
    sg = torch.empty((n, I, H // GROUP), dtype=torch.bfloat16, device=device)
    bg = torch.empty_like(sg)
    wu, su, bu = torch.empty_like(wg), torch.empty_like(sg), torch.empty_like(sg)
    wd = torch.empty((n, H, I // 8), dtype=torch.int32, device=device)
    sd = torch.empty((n, H, I // GROUP), dtype=torch.bfloat16, device=device)
    bd = torch.empty_like(sd)
    for j, e in enumerate(experts):
        base = (seed, w.name, layer, e)
        for (pw, ps, pb, N, K, tag) in ((wg, sg, bg, I, H, "gate"), (wu, su, bu, I, H, "up"), (wd, sd, bd, H, I, "down")):
            gen = torch_gen(device, *base, tag)
            m = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
            p, s, b = quantize_q4_g64(m)
            pw[j], ps[j], pb[j] = p, s, b
            del m, p, s, b
    return Bank(wg, sg, bg, wu, su, bu, wd, sd, bd)


def make_layer_mx(w: Workload, L: int, layer: int, seed: int = 0, device="cpu") -> LayerInput:
    """As :func:`make_layer` (compact) with an mxfp4 gs32 bank: same routes,
    router weights and activations; expert e's bytes depend only on
    (seed, layer, e)."""
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    used, remap = compact_ids(ids)
    parts = []
    for e in used.tolist():
        parts.append(gen_bank_mx(1, w.H, w.I, (seed, w.name, layer, int(e), "mx"), device))
    bank = BankMX(*[torch.cat([getattr(b, f) for b in parts]) for f in ("wg", "sg", "wu", "su", "wd", "sd")])
    return LayerInput(x=x, ids=remap, weights=tw, bank=bank, global_ids=ids)


def make_chain_layer(w: Workload, L: int, layer: int, seed: int = 0, device="cuda",
                     experts_per_chunk: int = 16) -> LayerInput:
    """One layer of a benchmark chain: compact bank of the used experts, each
    matrix drawn with one generator per (layer, matrix) in large chunks (fast
    on a GPU).  Same distributions as :func:`make_layer`; the bytes differ."""
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    used, remap = compact_ids(ids)
    bank = gen_bank(len(used), w.H, w.I, (seed, w.name, L, layer, "chain"), device, experts_per_chunk)
    return LayerInput(x=x, ids=remap, weights=tw, bank=bank, global_ids=ids)


def make_chain_layer_mx(w: Workload, L: int, layer: int, seed: int = 0, device="cuda",
                        experts_per_chunk: int = 8) -> LayerInput:
    """:func:`make_chain_layer` with an mxfp4 gs32 bank (same routes, router
    weights and activations)."""
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    used, remap = compact_ids(ids)
    bank = gen_bank_mx(len(used), w.H, w.I, (seed, w.name, L, layer, "chain-mx"), device, experts_per_chunk)
    return LayerInput(x=x, ids=remap, weights=tw, bank=bank, global_ids=ids)


def tiny_layer(device="cpu") -> LayerInput:
    """The tiny configuration exactly: E=8, top-2, H=256, I=128, L=2, seed 0, full bank."""
    w = WORKLOADS["tiny"]
    return make_layer(w, 2, 0, seed=0, device=device, compact=False)


def random_problem(L: int, k: int, E: int, H: int, I: int, seed: int, device="cpu", dup: bool = False):
    """Small random problem with a full bank; ``dup`` allows repeated ids within a token."""
    rng = np_rng("random_problem", L, k, E, H, I, seed)
    if dup:
        ids = rng.integers(0, E, size=(L, k)).astype(np.int32)
    else:
        ids = routes_uniform(L, k, E, rng)
    tw = router_weights(L, k, rng)
    x = gen_x(L, H, ("random_problem", seed, L, H), device)
    bank = gen_bank(E, H, I, ("random_problem", seed, E, H, I), device)
    return x, ids, tw, bank


def random_problem_mx(L: int, k: int, E: int, H: int, I: int, seed: int, device="cpu", dup: bool = False):
    """As :func:`random_problem` with an mxfp4 gs32 bank."""
    rng = np_rng("random_problem_mx", L, k, E, H, I, seed)
    if dup:
        ids = rng.integers(0, E, size=(L, k)).astype(np.int32)
    else:
        ids = routes_uniform(L, k, E, rng)
    tw = router_weights(L, k, rng)
    x = gen_x(L, H, ("random_problem_mx", seed, L, H), device)
    bank = gen_bank_mx(E, H, I, ("random_problem_mx", seed, E, H, I), device)
    return x, ids, tw, bank


def random_problem_q(codec: str, L: int, k: int, E: int, H: int, I: int, seed: int, device="cpu",
                     dup: bool = False):
    """As :func:`random_problem` with a bank in ``codec``."""
    rng = np_rng("random_problem_q", codec, L, k, E, H, I, seed)
    if dup:
        ids = rng.integers(0, E, size=(L, k)).astype(np.int32)
    else:
        ids = routes_uniform(L, k, E, rng)
    tw = router_weights(L, k, rng)
    x = gen_x(L, H, ("random_problem_q", seed, L, H), device)
    bank = gen_bank_q(codec, E, H, I, ("random_problem_q", seed, E, H, I), device)
    return x, ids, tw, bank


def make_layer_q(codec: str, w: Workload, L: int, layer: int, seed: int = 0, device="cpu") -> LayerInput:
    """As :func:`make_layer_mx` for any codec: expert e's bytes depend only on
    (seed, layer, e, codec)."""
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    used, remap = compact_ids(ids)
    parts = [gen_bank_q(codec, 1, w.H, w.I, (seed, w.name, layer, int(e)), device) for e in used.tolist()]
    ts = [None if parts[0].tensors()[i] is None else torch.cat([b.tensors()[i] for b in parts]) for i in range(9)]
    return LayerInput(x=x, ids=remap, weights=tw, bank=BankQ(codec, *ts), global_ids=ids)


def make_chain_layer_q(codec: str, w: Workload, L: int, layer: int, seed: int = 0, device="cuda",
                       experts_per_chunk: int = 8) -> LayerInput:
    """:func:`make_chain_layer` with a bank in ``codec``."""
    ids, tw = layer_routes(w, L, layer, seed)
    x = gen_x(L, w.H, (seed, w.name, L, layer), device)
    used, remap = compact_ids(ids)
    bank = gen_bank_q(codec, len(used), w.H, w.I, (seed, w.name, L, layer, "chain"), device, experts_per_chunk)
    return LayerInput(x=x, ids=remap, weights=tw, bank=bank, global_ids=ids)
