"""Inputs with tiny, zero and saturated activations for the parity tests.

Rewrites four tokens of a problem so that the hidden vectors of their pairs
sit far below fp32's usual range (about 1e-36), are zero, or come from gates
so negative that silu underflows.  Every value stays finite and the oracle's
results are finite; the cases check that no step of a path forms a scale
factor that overflows on such inputs.
"""

import numpy as np
import torch

ALL_CODECS = ["affine4_g64", "affine4_g32", "nvfp4", "mxfp4", "affine8_g64", "mxfp8"]


def gate_minus_one(bank, e):
    """Makes every gate weight of expert e equal to -1 (exactly, in any codec)."""
    c = bank.codec
    if c.startswith("affine"):
        bank.wg[e].zero_()
        bank.sg[e].zero_()
        bank.bg[e].fill_(-1.0)
    elif c in ("mxfp4", "nvfp4"):
        bank.wg[e].fill_(np.int32(np.uint32(0xAAAAAAAA).view(np.int32)))  # E2M1 code 0xA = -1.0
        bank.sg[e].fill_(127 if c == "mxfp4" else 0x38)                     # 2^0 / E4M3 1.0
    else:  # mxfp8
        bank.wg[e].fill_(np.int32(np.uint32(0xB8B8B8B8).view(np.int32)))   # E4M3 0xB8 = -1.0
        bank.sg[e].fill_(127)


def tiny_zero_saturated(x, ids, tw, bank, e_star):
    """Rewrites four tokens of a problem:
    token 0: x * 2^-66 (exact in bf16), so every h of its pairs is ~1e-37;
    token 1: x = 0;
    token 2: |x| scaled to sum 95, routed to e_star (gate weights all -1), so
             that pair's gates are all about -95 and silu underflows to 0;
    token 3: |x| scaled to sum 86, all its router weight on e_star: gates
             about -86, h about 1e-36, and the row is that pair alone."""
    x = x.clone()
    ids, tw = ids.copy(), tw.copy()
    x[0] = (x[0].float() * 2.0 ** -66).to(torch.bfloat16)
    x[1] = 0
    for t, s in ((2, 95.0), (3, 86.0)):
        a = x[t].float().abs()
        x[t] = (a * (s / a.sum())).to(torch.bfloat16)
        if e_star not in ids[t]:
            ids[t, 0] = e_star
    j = int(np.nonzero(ids[3] == e_star)[0][0])
    tw[3] = 0.0
    tw[3, j] = 1.0
    gate_minus_one(bank, e_star)
    return x, ids, tw
