"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test is chosen so that a plausible mistake in the oracle (nibble order,
scale/bias roles, gate/up swapped, a dropped combine weight, an index slip)
fails at least one of them:

* a hand-written word pattern fixes the nibble order;
* integer scale/bias fix the affine roles;
* quantize -> dequantize round trips fix the encoding against the generator;
* E=1, k=1, w=1 reduces the layer to a dense SwiGLU MLP checked against a
  library matmul;
* a multi-expert, multi-token brute force built from integer codes (never
  unpacked) checks the gather and the combine against a library matmul;
* a closed form with saturated SiLU gives exact integers;
* an asymmetric gate/up case fixes which projection goes through SiLU;
* invariances (router-weight scaling, slot permutation, expert relabelling).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def bf16_bits(vals) -> np.ndarray:
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_round(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def make_bank_from_codes(qg, sgv, bgv, qu, suv, buv, qd, sdv, bdv):
    """Bank from integer codes and float scale/bias arrays (already bf16-exact)."""
    def enc(q, s, b):
        q = torch.as_tensor(q, dtype=torch.int64)
        return (synth.pack_codes(q), torch.as_tensor(s, dtype=torch.float32).to(torch.bfloat16),
                torch.as_tensor(b, dtype=torch.float32).to(torch.bfloat16))
    return synth.Bank(*enc(qg, sgv, bgv), *enc(qu, suv, buv), *enc(qd, sdv, bdv))


def dense_from_codes(q, s, b):
    """Dense float64 matrix w[..., n, c] = s[..., n, c // 64] * q[..., n, c] + b[..., n, c // 64]."""
    s_full = np.repeat(np.asarray(s, np.float64), 64, axis=-1)
    b_full = np.repeat(np.asarray(b, np.float64), 64, axis=-1)
    return s_full * np.asarray(q, np.float64) + b_full


# --------------------------------------------------------------------------
# storage format
# --------------------------------------------------------------------------

def test_nibble_order_known_pattern():
    # Reading of the storage format: element c is nibble c % 8 of word c // 8,
    # lowest nibble first, so 0x76543210 holds 0, 1, ..., 7.
    words = np.array([[0x76543210, 0xFEDCBA98] * 4], dtype=np.uint32)  # one row, K = 64
    s = bf16_bits([1.0])
    b = bf16_bits([0.0])
    w = oracle.dequant(words, s.reshape(1, 1), b.reshape(1, 1))
    assert w.shape == (1, 64)
    assert list(w[0, :16]) == list(range(16))
    assert list(w[0, 16:32]) == list(range(16))


def test_scale_bias_roles_and_group_axis():
    # Two groups along K with different (scale, bias): w = s * q + b per group.
    q = np.arange(128) % 16
    words = synth.pack_codes(torch.tensor(q).reshape(1, 128)).numpy().view(np.uint32)
    s = bf16_bits([2.0, -0.5]).reshape(1, 2)
    b = bf16_bits([-3.0, 10.0]).reshape(1, 2)
    w = oracle.dequant(words, s, b)[0]
    assert np.array_equal(w[:64], 2.0 * q[:64] - 3.0)
    assert np.array_equal(w[64:], -0.5 * q[64:] + 10.0)


def test_pack_matches_hand_pattern():
    q = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7, 15, 14, 13, 12, 11, 10, 9, 8]])
    words = synth.pack_codes(q).numpy().view(np.uint32)
    assert words.tolist() == [[0x76543210, 0x89ABCDEF]]


# --------------------------------------------------------------------------
# quantize / dequantize round trip (generator vs oracle)
# --------------------------------------------------------------------------

def test_quantize_roundtrip_error_bound_and_requant():
    g = torch.Generator().manual_seed(1234)
    w = torch.randn((37, 256), generator=g).to(torch.bfloat16)
    packed, s, b = synth.quantize_q4_g64(w)
    deq = oracle.dequant(packed, s, b)
    wf = w.double().numpy()
    sf = np.repeat(s.double().numpy(), 64, axis=1)
    bf = np.repeat(b.double().numpy(), 64, axis=1)
    q = np.rint((deq - bf) / np.where(sf > 0, sf, 1.0))
    assert ((q >= 0) & (q <= 15)).all()
    # requantizing the dequantized values with the same (scale, bias) gives the codes back
    assert np.array_equal(deq, sf * q + bf)
    # elements whose code was not clamped sit within half a step of the input
    raw = (wf - bf) / sf
    unclamped = (raw > -0.5) & (raw < 15.5)
    err = np.abs(wf - deq)
    tol = sf / 2 * (1 + 2.0 ** -7) + 1e-30
    assert (err[unclamped] <= tol[unclamped]).all()
    # every element stays within one step (clamped ones only lose the bf16 rounding of the scale)
    assert (err <= sf * 1.05 + 1e-30).all()


def test_degenerate_group_is_exact():
    w = torch.full((2, 64), 0.75).to(torch.bfloat16)
    w[1] = -2.5
    packed, s, b = synth.quantize_q4_g64(w)
    assert (s.float() == 0).all()
    deq = oracle.dequant(packed, s, b)
    assert np.array_equal(deq, w.double().numpy())


# --------------------------------------------------------------------------
# the layer against library routines
# --------------------------------------------------------------------------

def _rand_codes(rng, shape_rows, K):
    q = rng.integers(0, 16, size=(*shape_rows, K))
    s = bf16_round(rng.uniform(0.05, 0.4, size=(*shape_rows, K // 64)))
    b = bf16_round(rng.uniform(-2.5, -0.5, size=(*shape_rows, K // 64)))
    return q, s, b


def test_dense_swiglu_special_case_matches_library():
    # E = 1, k = 1, router weight 1: the layer is a dense SwiGLU MLP.
    rng = np.random.default_rng(7)
    H, I, L = 192, 128, 3
    qg, sg, bg = _rand_codes(rng, (1, I), H)
    qu, su, bu = _rand_codes(rng, (1, I), H)
    qd, sd, bd = _rand_codes(rng, (1, H), I)
    bank = make_bank_from_codes(qg, sg, bg, qu, su, bu, qd, sd, bd)
    x = torch.randn((L, H), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    ids = np.zeros((L, 1), np.int32)
    tw = np.ones((L, 1), np.float32)
    out = oracle.forward_pairs(x, ids, tw, bank)

    Wg = torch.from_numpy(dense_from_codes(qg, sg, bg)[0])
    Wu = torch.from_numpy(dense_from_codes(qu, su, bu)[0])
    Wd = torch.from_numpy(dense_from_codes(qd, sd, bd)[0])
    xd = x.double()
    ref = torch.nn.functional.linear(torch.nn.functional.silu(xd @ Wg.T) * (xd @ Wu.T), Wd).numpy()
    rel = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_multi_expert_brute_force_matches_library(seed):
    # Several experts and tokens, router weights, duplicate ids allowed.
    rng = np.random.default_rng(100 + seed)
    E, H, I, L, k = 5, 128, 64, 4, 3
    qg, sg, bg = _rand_codes(rng, (E, I), H)
    qu, su, bu = _rand_codes(rng, (E, I), H)
    qd, sd, bd = _rand_codes(rng, (E, H), I)
    bank = make_bank_from_codes(qg, sg, bg, qu, su, bu, qd, sd, bd)
    x = torch.from_numpy(rng.standard_normal((L, H)).astype(np.float32)).to(torch.bfloat16)
    ids = rng.integers(0, E, size=(L, k)).astype(np.int32)
    ids[0, 1] = ids[0, 0]  # a duplicate slot
    tw = rng.uniform(0.1, 1.0, size=(L, k)).astype(np.float32)
    out = oracle.forward_pairs(x, ids, tw, bank)

    Wg = torch.from_numpy(dense_from_codes(qg, sg, bg))
    Wu = torch.from_numpy(dense_from_codes(qu, su, bu))
    Wd = torch.from_numpy(dense_from_codes(qd, sd, bd))
    xd = x.double()
    ref = torch.zeros((L, H), dtype=torch.float64)
    for t in range(L):
        for j in range(k):
            e = int(ids[t, j])
            h = torch.nn.functional.silu(Wg[e] @ xd[t]) * (Wu[e] @ xd[t])
            ref[t] += float(tw[t, j]) * (Wd[e] @ h)
    ref = ref.numpy()
    rel = np.linalg.norm(out - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert rel.max() < 1e-12


def test_fp32_library_computation_within_fp32_bound():
    # The double oracle and a float32 library evaluation of the same layer
    # agree to the float32 rounding scale (far inside the 1e-3 contract).
    x, ids, tw, bank = synth.random_problem(3, 2, 6, 256, 128, seed=5)
    out = oracle.forward_pairs(x, ids, tw, bank)
    dg = torch.from_numpy(oracle.dequant(bank.wg, bank.sg, bank.bg)).float()
    du = torch.from_numpy(oracle.dequant(bank.wu, bank.su, bank.bu)).float()
    dd = torch.from_numpy(oracle.dequant(bank.wd, bank.sd, bank.bd)).float()
    xf = x.float()
    ref = torch.zeros((3, 256))
    for t in range(3):
        for j in range(2):
            e = int(ids[t, j])
            h = torch.nn.functional.silu(dg[e] @ xf[t]) * (du[e] @ xf[t])
            ref[t] += float(tw[t, j]) * (dd[e] @ h)
    rel = np.linalg.norm(out - ref.double().numpy(), axis=1) / np.linalg.norm(out, axis=1)
    assert rel.max() < 1e-5


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_closed_form_saturated_silu_integers():
    # x = 1, every gate weight 1 * 1 + 0.5625 -> gate = 64 * 1.5625 = 100, so
    # silu(gate) = 100 exactly in double (exp(-100) vanishes against 1);
    # every up weight 0.5 * 3 = 1.5 -> up = 96; h = 9600 on every hidden row.
    # Down weights: code (m % 16) with scale 1/64 and bias 0 in row m, so
    # y[m] = 64 * 9600 * (m % 16) / 64 = 9600 * (m % 16).  Expert 1 doubles
    # the down scale.  Router weights 0.5 / 0.25 -> exact sums.
    H = I = 64
    E = 2
    qg = np.ones((E, I, H), np.int64)
    sg = np.ones((E, I, 1))
    bg = np.full((E, I, 1), 0.5625)
    qu = np.full((E, I, H), 3)
    su = np.full((E, I, 1), 0.5)
    bu = np.zeros((E, I, 1))
    qd = np.broadcast_to((np.arange(H) % 16)[None, :, None], (E, H, I)).copy()
    sd = np.stack([np.full((H, 1), 1 / 64), np.full((H, 1), 2 / 64)])
    bd = np.zeros((E, H, 1))
    bank = make_bank_from_codes(qg, sg, bg, qu, su, bu, qd, sd, bd)
    x = torch.ones((2, H)).to(torch.bfloat16)
    ids = np.array([[0, 1], [1, 1]], np.int32)
    tw = np.array([[0.5, 0.25], [0.5, 0.25]], np.float32)
    out = oracle.forward_pairs(x, ids, tw, bank)
    m = np.arange(H) % 16
    assert np.array_equal(out[0], 9600.0 * m * (0.5 * 1 + 0.25 * 2))
    assert np.array_equal(out[1], 9600.0 * m * (0.5 * 2 + 0.25 * 2))
    assert np.array_equal(oracle.forward_union(x, ids, tw, bank), out)


def test_gate_goes_through_silu_not_up():
    # gate = -60, up = +60: silu(-60) * 60 is ~1e-22; with the roles swapped the
    # result would be silu(60) * (-60) = -3600 per hidden row.
    H = I = 64
    qg = np.zeros((1, I, H), np.int64)
    sg = np.ones((1, I, 1))
    bg = np.full((1, I, 1), -60 / 64)
    qu = np.zeros((1, I, H), np.int64)
    su = np.ones((1, I, 1))
    bu = np.full((1, I, 1), 60 / 64)
    qd = np.ones((1, H, I), np.int64)
    sd = np.ones((1, H, 1))
    bd = np.zeros((1, H, 1))
    bank = make_bank_from_codes(qg, sg, bg, qu, su, bu, qd, sd, bd)
    x = torch.ones((1, H)).to(torch.bfloat16)
    out = oracle.forward_pairs(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), bank)
    h = -60.0 / (1.0 + math.exp(60.0)) * 60.0
    assert np.allclose(out, I * h, rtol=1e-12, atol=0)
    assert np.abs(out).max() < 1e-18


def test_silu_overflow_gives_signed_zero_not_nan():
    H = I = 64
    bank = make_bank_from_codes(np.zeros((1, I, H)), np.ones((1, I, 1)), np.full((1, I, 1), -1000 / 64),
                                np.zeros((1, I, H)), np.ones((1, I, 1)), np.ones((1, I, 1)),
                                np.ones((1, H, I)), np.ones((1, H, 1)), np.zeros((1, H, 1)))
    x = torch.ones((1, H)).to(torch.bfloat16)
    out = oracle.forward_pairs(x, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), bank)
    assert np.isfinite(out).all() and (out == 0).all()


# --------------------------------------------------------------------------
# invariances and the two evaluation modes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dup", [False, True])
def test_union_mode_equals_pair_mode(dup):
    x, ids, tw, bank = synth.random_problem(5, 3, 7, 128, 64, seed=11, dup=dup)
    a = oracle.forward_pairs(x, ids, tw, bank)
    b = oracle.forward_union(x, ids, tw, bank)
    rel = np.linalg.norm(a - b, axis=1) / np.linalg.norm(a, axis=1)
    assert rel.max() < 1e-13


def test_router_weight_scaling_is_exact():
    x, ids, tw, bank = synth.random_problem(3, 2, 5, 128, 64, seed=12)
    a = oracle.forward_pairs(x, ids, tw, bank)
    b = oracle.forward_pairs(x, ids, tw * np.float32(2), bank)
    assert np.array_equal(b, 2 * a)


def test_slot_permutation_invariance():
    x, ids, tw, bank = synth.random_problem(4, 4, 9, 128, 64, seed=13)
    a = oracle.forward_pairs(x, ids, tw, bank)
    perm = np.array([2, 0, 3, 1])
    b = oracle.forward_pairs(x, ids[:, perm], tw[:, perm], bank)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-9)


def test_expert_relabel_invariance():
    x, ids, tw, bank = synth.random_problem(3, 2, 6, 128, 64, seed=14)
    a = oracle.forward_pairs(x, ids, tw, bank)
    relabel = np.array([4, 2, 5, 0, 1, 3])  # old expert e -> new id relabel[e]
    order = np.argsort(relabel)             # new id -> old expert
    b = oracle.forward_pairs(x, relabel[ids].astype(np.int32), tw, bank.select(order))
    assert np.array_equal(a, b)


def test_single_output_element_matches_full():
    x, ids, tw, bank = synth.random_problem(3, 2, 6, 128, 64, seed=15)
    full = oracle.forward_pairs(x, ids, tw, bank)
    for (t, m) in [(0, 0), (1, 77), (2, 127)]:
        assert oracle.output_element(x, ids, tw, bank, t, m) == full[t, m]


def test_tiny_configuration_runs_and_is_finite():
    lay = synth.tiny_layer()
    out = oracle.forward_pairs(lay.x, lay.ids, lay.weights, lay.bank)
    assert out.shape == (2, 256) and np.isfinite(out).all()
    assert np.array_equal(oracle.forward_union(lay.x, lay.ids, lay.weights, lay.bank), out)


def test_invalid_ids_are_rejected():
    x, ids, tw, bank = synth.random_problem(2, 2, 4, 64, 64, seed=16)
    bad = ids.copy()
    bad[1, 0] = 4
    with pytest.raises(oracle.OracleError):
        oracle.forward_pairs(x, bad, tw, bank)
    bad[1, 0] = -1
    with pytest.raises(oracle.OracleError):
        oracle.forward_union(x, bad, tw, bank)
    with pytest.raises(oracle.OracleError):
        oracle.route_union(bad, tw, 4)


def test_thread_count_does_not_change_results():
    x, ids, tw, bank = synth.random_problem(3, 2, 5, 128, 64, seed=17)
    n = oracle.threads()
    oracle.set_threads(1)
    a = oracle.forward_pairs(x, ids, tw, bank)
    oracle.set_threads(max(2, n))
    b = oracle.forward_pairs(x, ids, tw, bank)
    oracle.set_threads(n)
    assert np.array_equal(a, b)
