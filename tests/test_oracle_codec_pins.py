"""Pins of the CPU oracle's further codecs (no GPU needed).

The pages name these storage modes without their bit layouts: mxfp8 (the
dequant-mode comparison of the mlx discussion "Small-L fused expert gather
for fine-grained MoE decode"), nvfp4 and mxfp8 (PR 4572 on the page "MoE
GatherQMM small-M verify cost", Facts), 8-bit affine models (that page's
correctness reports) and affine with group 32 (the same dequant-mode
comparison).  The oracle takes the OCP encodings for the float formats and
the affine recipe of the 4-bit banks for the integer ones.  A plausible
mistake -- an exponent bias, a subnormal step, a lost NaN, a byte shift, a
block size, a group index -- fails at least one of:

* every E4M3 byte decodes to the value PyTorch's float8_e4m3fn gives it (a
  library routine), NaNs at the same codes;
* known 8-bit and 4-bit code patterns decode in order with unit scale;
* a group-64 affine bank re-expressed with group 32 (each scale and bias
  repeated) is the same matrix, and a group-32 bank whose halves differ is
  not a group-64 one;
* an nvfp4 scale byte multiplies exactly its own 16 inputs by its E4M3
  value, an mxfp8 scale byte 127 + n exactly its own 32 inputs by 2^n;
* values built on each codec's grid survive the generator's encoder and the
  oracle's decoder exactly;
* each codec's layer equals library matmuls over its dense dequantized
  weights, the union evaluation equals the per-pair one, single elements
  equal the full evaluation, and the generic entry agrees with the 4-bit
  affine and mxfp4 ones;
* an mxfp8 bank is about twice the bytes of an mxfp4 bank (the pages).
"""

import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CODECS = sorted(oracle.CODECS)


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = float(v)
    return vals


def test_e4m3_decoder_matches_library_float8():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle.e4m3_value(b) for b in range(256)])
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    assert np.isnan(ours).sum() == 2
    fin = ~np.isnan(lib)
    assert np.array_equal(ours[fin], lib[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(lib[fin]))
    assert ours[126] == 448.0 and ours[1] == 2.0 ** -9 and ours[8] == 2.0 ** -6


def _one_row(codec, codes, scale_val):
    """Packed words and unit-ish scales for one row of the given codes."""
    bits, gs, bias = synth.CODECS[codec]
    K = len(codes)
    q = torch.as_tensor(codes, dtype=torch.int64).reshape(1, K)
    w = synth.pack_codes8(q) if bits == 8 else synth.pack_codes(q)
    if bias:
        s = torch.full((1, K // gs), scale_val, dtype=torch.bfloat16)
        b = torch.zeros((1, K // gs), dtype=torch.bfloat16)
        return w, s, b
    return w, torch.full((1, K // gs), scale_val, dtype=torch.uint8), None


def test_known_code_patterns_decode_in_order():
    # 8-bit affine: word 0x03020100 holds codes 0, 1, 2, 3 (lowest byte first)
    w = np.array([[0x03020100, 0x07060504] + [0] * 14], np.uint32)
    s = torch.ones((1, 1), dtype=torch.bfloat16)
    b = torch.zeros((1, 1), dtype=torch.bfloat16)
    got = oracle.dequant_q("affine8_g64", w, s, b)[0]
    assert np.array_equal(got[:8], np.arange(8.0)) and not got[8:].any()
    # 4-bit affine group 32: nibbles lowest first
    w4 = np.array([[0x76543210, 0xFEDCBA98, 0, 0]], np.uint32)
    got4 = oracle.dequant_q("affine4_g32", w4, torch.ones((1, 1), dtype=torch.bfloat16),
                            torch.zeros((1, 1), dtype=torch.bfloat16))[0]
    assert np.array_equal(got4[:16], np.arange(16.0))
    # mxfp8 with scale 2^0: byte b decodes as the E4M3 value of b
    codes = list(range(0, 126, 4))[:32]
    w8, s8, _ = _one_row("mxfp8", codes, 127)
    got8 = oracle.dequant_q("mxfp8", w8, s8)[0]
    ref = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got8, ref)


def test_affine_group32_is_group64_with_repeated_scales():
    torch.manual_seed(0)
    m = torch.randn(3, 128).to(torch.bfloat16)
    for bits in (4, 8):
        w64, s64, b64 = synth.quantize_affine(m, bits, 64)
        s32 = s64.repeat_interleave(2, dim=-1)
        b32 = b64.repeat_interleave(2, dim=-1)
        d64 = oracle.dequant_q(f"affine{bits}_g64", w64, s64, b64)
        d32 = oracle.dequant_q(f"affine{bits}_g32", w64, s32, b32)
        assert np.array_equal(d64, d32)
        # halves with their own scale: changing one half's scale moves only that half
        s32b = s32.clone()
        s32b[:, 1] = s32b[:, 1] * 2
        d32b = oracle.dequant_q(f"affine{bits}_g32", w64, s32b, b32)
        q = (d32[:, 32:64] - b32[:, 1:2].double().numpy()) / s32[:, 1:2].double().numpy()
        assert np.allclose(d32b[:, 32:64], q * 2 * s32[:, 1:2].double().numpy() + b32[:, 1:2].double().numpy())
        assert np.array_equal(d32b[:, :32], d32[:, :32]) and np.array_equal(d32b[:, 64:], d32[:, 64:])


def test_block_scales_act_on_their_own_block():
    rng = np.random.default_rng(2)
    # nvfp4: scale code c multiplies its 16 inputs by e4m3(c)
    codes = rng.integers(0, 16, size=64)
    w, _, _ = _one_row("nvfp4", codes, 0)
    one = 0x38  # E4M3 1.0
    base = oracle.dequant_q("nvfp4", w, np.full((1, 4), one, np.uint8))[0]
    for c in (0x01, 0x30, 0x3C, 0x45, 0x7E, 0xB8):
        sc = np.full((1, 4), one, np.uint8)
        sc[0, 2] = c
        got = oracle.dequant_q("nvfp4", w, sc)[0]
        f = torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        assert np.array_equal(got[32:48], base[32:48] * f)
        assert np.array_equal(np.delete(got, np.s_[32:48]), np.delete(base, np.s_[32:48]))
    # mxfp8: scale byte 127 + n multiplies its 32 inputs by 2^n; 255 is NaN
    codes8 = rng.integers(0, 126, size=64)
    w8, _, _ = _one_row("mxfp8", codes8, 127)
    base8 = oracle.dequant_q("mxfp8", w8, np.full((1, 2), 127, np.uint8))[0]
    for n in (-20, -3, 2, 9):
        got = oracle.dequant_q("mxfp8", w8, np.array([[127, 127 + n]], np.uint8))[0]
        assert np.array_equal(got[32:], base8[32:] * 2.0 ** n) and np.array_equal(got[:32], base8[:32])
    nan = oracle.dequant_q("mxfp8", w8, np.array([[255, 127]], np.uint8))[0]
    assert np.isnan(nan[:32]).all() and np.array_equal(nan[32:], base8[32:])


def test_grid_values_roundtrip_through_encoders_and_decoder():
    rng = np.random.default_rng(3)
    N, K = 4, 64
    e2m1 = np.array(synth.E2M1_MAGNITUDES)
    # nvfp4: E2M1 grid values times a per-16 E4M3 scale, block maximum 6 * scale
    vals = np.empty((N, K))
    for r in range(N):
        for b in range(K // 16):
            sc = 2.0 ** int(rng.integers(-6, 3))
            mag = rng.choice(e2m1, size=16)
            mag[rng.integers(0, 16)] = 6.0
            vals[r, 16 * b:16 * (b + 1)] = mag * rng.choice([1.0, -1.0], size=16) * sc
    w = torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(w.float().numpy(), vals)
    p, s, _ = synth.quantize_nvfp4_g16(w)
    assert np.array_equal(oracle.dequant_q("nvfp4", p, s), vals)
    # mxfp8: E4M3 grid values with a block maximum in [256, 448], times 2^n
    grid = synth.e4m3_grid().numpy()
    vals8 = np.empty((N, K))
    for r in range(N):
        for b in range(K // 32):
            mag = rng.choice(grid[grid <= 448], size=32)
            mag[rng.integers(0, 32)] = rng.choice(grid[grid >= 256])
            vals8[r, 32 * b:32 * (b + 1)] = mag * rng.choice([1.0, -1.0], size=32) * 2.0 ** int(rng.integers(-8, 4))
    w8 = torch.tensor(vals8, dtype=torch.float32).to(torch.bfloat16)
    keep = np.array_equal(w8.float().numpy(), vals8)  # E4M3 values have 4 significant bits: bf16-exact
    assert keep
    p8, s8, _ = synth.quantize_mxfp8_g32(w8)
    assert np.array_equal(oracle.dequant_q("mxfp8", p8, s8), vals8)
    # affine: integer codes with exact scale and bias survive
    for bits in (4, 8):
        lv = (1 << bits) - 1
        q = rng.integers(0, lv + 1, size=(N, K))
        q[:, 0::32], q[:, 1::32] = 0, lv  # every group spans the full code range
        sv, bv = 0.125, -2.5
        wa = torch.tensor(q * sv + bv, dtype=torch.float32).to(torch.bfloat16)
        pa, sa, ba = synth.quantize_affine(wa, bits, 32)
        assert np.array_equal(oracle.dequant_q(f"affine{bits}_g32", pa, sa, ba), q * sv + bv)


@pytest.mark.parametrize("codec", CODECS)
def test_layer_equals_library_matmul_over_dense_weights(codec):
    L, k, E, H, I = 3, 3, 5, 128, 96 if codec != "affine4_g64" and codec != "affine8_g64" else 128
    x, ids, tw, bank = synth.random_problem_q(codec, L, k, E, H, I, seed=4)
    ref = oracle.forward_pairs_q(codec, x, ids, tw, bank)
    xf = x.float().numpy().astype(np.float64)
    Wg = oracle.dequant_q(codec, bank.wg, bank.sg, bank.bg)
    Wu = oracle.dequant_q(codec, bank.wu, bank.su, bank.bu)
    Wd = oracle.dequant_q(codec, bank.wd, bank.sd, bank.bd)
    g = torch.from_numpy(Wg[ids]) @ torch.from_numpy(xf)[:, None, :, None]
    u = torch.from_numpy(Wu[ids]) @ torch.from_numpy(xf)[:, None, :, None]
    h = (g / (1.0 + torch.exp(-g)) * u)
    y = (torch.from_numpy(Wd[ids]) @ h)[..., 0]
    out = (y * torch.from_numpy(tw.astype(np.float64))[..., None]).sum(1).numpy()
    assert np.allclose(ref, out, rtol=1e-10, atol=1e-9 * np.abs(out).max())


@pytest.mark.parametrize("codec", CODECS)
def test_union_single_element_and_generic_entry(codec):
    x, ids, tw, bank = synth.random_problem_q(codec, 4, 3, 6, 64, 128, seed=5, dup=True)
    a = oracle.forward_pairs_q(codec, x, ids, tw, bank)
    b = oracle.forward_union_q(codec, x, ids, tw, bank)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(a).max())
    for t, m in ((0, 0), (3, 63), (2, 17)):
        assert oracle.output_element_q(codec, x, ids, tw, bank, t, m) == pytest.approx(a[t, m], rel=1e-12,
                                                                                      abs=1e-12)
    if codec == "affine4_g64":
        legacy = synth.Bank(*bank.tensors())
        assert np.array_equal(oracle.forward_pairs(x, ids, tw, legacy), a)
    if codec == "mxfp4":
        legacy = synth.BankMX(bank.wg, bank.sg, bank.wu, bank.su, bank.wd, bank.sd)
        assert np.array_equal(oracle.forward_pairs_mx(x, ids, tw, legacy), a)


def test_invalid_codec_shapes_are_rejected():
    x, ids, tw, bank = synth.random_problem_q("nvfp4", 2, 2, 3, 64, 32, seed=6)
    with pytest.raises(oracle.OracleError):  # H = 56 is not a multiple of 16
        oracle.forward_pairs_q("nvfp4", x[:, :56], ids, tw, synth.BankQ(
            "nvfp4", bank.wg[:, :, :7], bank.sg[:, :, :3], None, bank.wu[:, :, :7], bank.su[:, :, :3], None,
            bank.wd, bank.sd, None))
    with pytest.raises(oracle.OracleError):  # affine without biases
        oracle.forward_pairs_q("affine8_g32", *synth.random_problem_q("mxfp8", 2, 2, 3, 64, 32, seed=6)[:3],
                               synth.random_problem_q("mxfp8", 2, 2, 3, 64, 32, seed=6)[3])


def test_mxfp8_is_twice_the_bytes_of_mxfp4():
    g = _golden("mxfp8_bytes_ratio.txt")
    H, I = 6144, 2048
    b4 = 3 * (H * I // 2 + H * I // 32)
    b8 = 3 * (H * I + H * I // 32)
    assert abs(b8 / b4 - g["ratio_printed"]) < 0.1
