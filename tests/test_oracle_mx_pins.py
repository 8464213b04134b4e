"""Pins of the CPU oracle's mxfp4 gs32 evaluation (no GPU needed).

The pages name the format (GLM-5.2's mxfp4 gs32 banks, about 20 MB per
expert) without its bit layouts; the oracle follows the OCP MX v1.0 encodings
(FP4 E2M1 elements, E8M0 power-of-two block scales).  A plausible mistake --
exponent bias, mantissa weight, sign bit, nibble order, scale bias or block
size -- fails at least one of these:

* the byte count of one expert matches the pages' ~20 MB;
* the decoded code table has the E2M1 closed-form properties: 16 codes, 8
  distinct magnitudes whose largest is 6, sign symmetry by bit 3, subnormal
  step 0.5, each binade [2^e, 2^(e+1)) holding two values one half-step apart;
* a scale byte of 127 + n multiplies a whole 32-input block by 2^n and leaves
  the neighbouring block alone;
* values built on the E2M1 grid survive the generator's quantizer (an
  independent table-based encoder) and the oracle's decoder exactly;
* the layer over an mxfp4 bank equals a library matmul over its dense
  dequantized weights, and the union evaluation equals the per-pair one.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    return vals


def test_bytes_per_expert_matches_pages():
    g = _golden("mxfp4_bytes_per_expert.txt")
    H, I = int(g["H"]), int(g["I"])
    per_matrix = H * I // 2 + H * I // 32  # 4-bit elements + one byte per 32 inputs
    total = 3 * per_matrix
    assert abs(total / 1e6 - g["megabytes_printed"]) < 0.5


def _decode_all_codes(scale_byte=127):
    words = np.array([[0x76543210, 0xFEDCBA98, 0, 0]], np.uint32)
    return oracle.dequant_mx(words, np.array([[scale_byte]], np.uint8))[0, :16]


def test_code_table_closed_form_properties():
    v = _decode_all_codes()
    mags = v[:8]
    assert np.all(v[8:] == -mags) and np.all(np.signbit(v[8:]))  # bit 3 is the sign
    assert len(set(mags.tolist())) == 8 and mags.max() == 6.0 and mags[0] == 0.0
    assert np.all(np.diff(mags) > 0)  # magnitude grows with the code
    assert mags[1] == 0.5  # subnormal step: 2^(1 - bias) * 2^-1 with bias 1
    # each exponent's binade holds the two mantissa values 1.0 and 1.5 times 2^e
    for e in range(3):
        lo, hi = mags[2 + 2 * e], mags[3 + 2 * e]
        assert lo == 2.0 ** e and hi == 1.5 * lo


def test_scale_byte_is_a_power_of_two_per_block():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=(2, 64))
    words = synth.pack_codes(torch.as_tensor(codes)).numpy().view(np.uint32)
    base = oracle.dequant_mx(words, np.array([[127, 127], [127, 127]], np.uint8))
    for n in (-9, -1, 1, 5):
        got = oracle.dequant_mx(words, np.array([[127 + n, 127], [127, 127 + n]], np.uint8))
        assert np.array_equal(got[0, :32], base[0, :32] * 2.0 ** n)
        assert np.array_equal(got[0, 32:], base[0, 32:])
        assert np.array_equal(got[1, :32], base[1, :32])
        assert np.array_equal(got[1, 32:], base[1, 32:] * 2.0 ** n)
    nan = oracle.dequant_mx(words, np.array([[255, 127], [127, 127]], np.uint8))
    assert np.isnan(nan[0, :32]).all() and np.array_equal(nan[0, 32:], base[0, 32:])


def test_grid_values_roundtrip_through_quantizer_and_decoder():
    rng = np.random.default_rng(1)
    grid = np.array(synth.E2M1_MAGNITUDES)
    N, K = 6, 128
    vals = np.empty((N, K))
    for r in range(N):
        for b in range(K // 32):
            mag = rng.choice(grid, size=32)
            mag[rng.integers(0, 32)] = 6.0 * rng.choice([1, -1])  # block maximum pins the exponent
            sign = rng.choice([1.0, -1.0], size=32)
            vals[r, 32 * b:32 * (b + 1)] = np.abs(mag) * np.where(mag < 0, -1.0, sign) * 2.0 ** int(rng.integers(-6, 4))
    w = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(w.float().numpy(), vals)  # bf16-exact by construction
    packed, scale = synth.quantize_mxfp4_g32(w)
    back = oracle.dequant_mx(packed, scale)
    assert np.array_equal(back, vals)


def test_layer_equals_library_matmul_over_dense_weights():
    x, ids, tw, bank = synth.random_problem_mx(4, 3, 6, 96, 160, seed=2)
    ref = oracle.forward_pairs_mx(x, ids, tw, bank)
    xf = x.float().numpy().astype(np.float64)
    Wg = oracle.dequant_mx(bank.wg, bank.sg)
    Wu = oracle.dequant_mx(bank.wu, bank.su)
    Wd = oracle.dequant_mx(bank.wd, bank.sd)
    out = np.zeros((4, 96))
    for t in range(4):
        for j in range(3):
            e = ids[t, j]
            g = Wg[e] @ xf[t]
            u = Wu[e] @ xf[t]
            h = g / (1.0 + np.exp(-g)) * u
            out[t] += float(tw[t, j]) * (Wd[e] @ h)
    assert np.allclose(ref, out, rtol=1e-10, atol=1e-9 * np.abs(out).max())


@pytest.mark.parametrize("dup", [False, True])
def test_union_mode_equals_pair_mode(dup):
    x, ids, tw, bank = synth.random_problem_mx(5, 4, 7, 64, 96, seed=3, dup=dup)
    a = oracle.forward_pairs_mx(x, ids, tw, bank)
    b = oracle.forward_union_mx(x, ids, tw, bank)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_output_element_matches_full():
    x, ids, tw, bank = synth.random_problem_mx(3, 2, 4, 64, 96, seed=4)
    full = oracle.forward_pairs_mx(x, ids, tw, bank)
    for t, m in ((0, 0), (2, 63), (1, 17)):
        assert oracle.output_element_mx(x, ids, tw, bank, t, m) == pytest.approx(full[t, m], rel=1e-12, abs=1e-12)


def test_shapes_not_multiple_of_32_are_rejected():
    x, ids, tw, bank = synth.random_problem_mx(2, 2, 3, 64, 96, seed=5)
    bad = synth.BankMX(bank.wg[:, :, :6], bank.sg[:, :, :1], bank.wu[:, :, :6], bank.su[:, :, :1],
                       bank.wd, bank.sd)  # H = 48
    with pytest.raises(oracle.OracleError):
        oracle.forward_pairs_mx(x[:, :48], ids, tw, bad)
