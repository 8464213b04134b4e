"""GPU parity of the union path against the CPU oracle (needs an MI355X).

Bars: union / index outputs bit-exact; fp32 layer outputs within a per-row
normwise relative error of 1e-3 (the contract), and within 6e-4, the bound
the kernels' arithmetic gives: gate and up accumulate exact bf16 products in
fp32 (about 1e-6 after the affine offset's cancellation), while the down
projection reads the hidden vector h rounded to fp16 after an exact
power-of-two scaling -- unit roundoff 2^-11 = 4.9e-4 per element, about
2^-11 / sqrt(3) = 2.8e-4 normwise with random-sign rounding errors; bf16
outputs equal the round-to-nearest-even of the fp32 outputs bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tiny_cases import ALL_CODECS, tiny_zero_saturated

pytestmark = pytest.mark.gpu

CONTRACT = 1e-3
ARITH = 6e-4


def _q():
    import quantized_expert_gather_amd as q
    return q


def say(*a):
    print("[case]", *a, flush=True)


def rel_err_rows(gpu: np.ndarray, ref: np.ndarray) -> np.ndarray:
    num = np.linalg.norm(gpu.astype(np.float64) - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def run_layer(x, ids, tw, bank, out_dtype=torch.float32, stages_split=False):
    q = _q()
    dev = torch.device("cuda")
    xd = x.to(dev)
    idd = torch.as_tensor(np.asarray(ids, np.int32)).to(dev)
    twd = torch.as_tensor(np.asarray(tw, np.float32)).to(dev)
    bk = bank.to(dev)
    L, k = idd.shape
    ws = q.new_workspace(L, k, bk.E, x.shape[1], bk.wg.shape[1], dev)
    if stages_split:
        out = torch.empty((L, x.shape[1]), dtype=out_dtype, device=dev)
        q.forward_bank(xd, idd, twd, bk, out=out, out_dtype=out_dtype, workspace=ws, stages=q.MOE_Q4_STAGE_GATEUP)
        q.forward_bank(xd, idd, twd, bk, out=out, out_dtype=out_dtype, workspace=ws, stages=q.MOE_Q4_STAGE_DOWN)
    else:
        out = q.forward_bank(xd, idd, twd, bk, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def check_layer(x, ids, tw, bank, label):
    say(label, "L=%d k=%d E=%d H=%d I=%d" % (ids.shape[0], ids.shape[1], bank.E, x.shape[1], bank.wg.shape[1]))
    ref = oracle.forward_pairs(x.cpu(), ids, tw, bank.to("cpu"))
    out, ws = run_layer(x, ids, tw, bank)
    got = out.float().cpu().numpy()
    err = rel_err_rows(got, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= CONTRACT
    assert err.max() <= ARITH
    status, path = _q().moe_q4_read_device_status(ws)
    assert status == 0 and path == _q().MOE_Q4_PATH_UNION
    return got, ref


# ---------------------------------------------------------------------------
# route union, bit-exact
# ---------------------------------------------------------------------------

UNION_CASES = {
    "random_L8": lambda rng: rng.integers(0, 256, size=(8, 8)),
    "all_same": lambda rng: np.full((4, 8), 17),
    "all_distinct": lambda rng: np.arange(64).reshape(8, 8)[:, ::-1],
    "dup_in_token": lambda rng: np.array([[3, 3, 5, 255], [255, 0, 0, 3]]),
    "last_id": lambda rng: np.full((3, 2), 255),
    "L32": lambda rng: rng.integers(0, 256, size=(32, 8)),
    "L1": lambda rng: rng.permutation(256)[:8].reshape(1, 8),
    "k1": lambda rng: rng.integers(0, 256, size=(7, 1)),
    "E288_L4": lambda rng: rng.integers(0, 288, size=(4, 8)),
    "E16384": lambda rng: rng.integers(0, 16384, size=(16, 8)),
    "pairs1024": lambda rng: rng.integers(0, 4096, size=(32, 32)),
}


@pytest.mark.parametrize("case", sorted(UNION_CASES))
def test_route_union_bit_exact(case):
    q = _q()
    rng = np.random.default_rng(abs(hash(case)) % 2**32)
    ids = np.asarray(UNION_CASES[case](rng), np.int32)
    E = {"E288_L4": 288, "E16384": 16384, "pairs1024": 4096}.get(case, 256)
    L, k = ids.shape
    tw = rng.uniform(0, 1, size=(L, k)).astype(np.float32)
    say("route_union", case, ids.shape, E)
    ref = oracle.route_union(ids, tw, E)
    r = q.moe_route_union(torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), E)
    torch.cuda.synchronize()
    u = int(r["u"].item())
    assert u == ref["u"]
    assert r["uniq_ids"][:u].cpu().numpy().tolist() == ref["uniq_ids"].tolist()
    assert (r["uniq_ids"][u:].cpu().numpy() == -1).all()
    assert np.array_equal(r["tok_mask"][:u].cpu().numpy().view(np.uint32), ref["tok_mask"])
    assert np.array_equal(r["uniq_w"][:u].cpu().numpy().view(np.uint32), ref["uniq_w"].view(np.uint32))
    assert (r["uniq_w"][u:].cpu().numpy() == 0).all()
    assert np.array_equal(r["slot_to_uniq"].cpu().numpy(), ref["slot_to_uniq"])


def test_route_union_invalid_ids_map_to_minus_one():
    q = _q()
    ids = np.array([[1, 300], [-5, 1]], np.int32)
    tw = np.ones((2, 2), np.float32)
    r = q.moe_route_union(torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), 256)
    torch.cuda.synchronize()
    assert int(r["u"].item()) == 1
    assert r["slot_to_uniq"].cpu().numpy().tolist() == [[0, -1], [-1, 0]]


# ---------------------------------------------------------------------------
# layer parity
# ---------------------------------------------------------------------------

def test_tiny_configuration():
    lay = synth.tiny_layer()
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, "tiny E8 k2 H256 I128 L2 seed0")


SMALL_SHAPES = [
    # (L, k, E, H, I, dup) -- ragged lane groups (H/32, I/32 not powers of two),
    # several row blocks, several positions per lane, duplicates
    (1, 2, 4, 64, 64, False),
    (3, 2, 6, 384, 192, False),
    (5, 3, 7, 320, 128, True),
    (8, 4, 16, 2048, 256, False),
    (4, 8, 12, 4096, 128, True),
    (2, 8, 64, 6144, 128, False),
    (7, 8, 40, 6144, 64, False),
    (16, 4, 40, 512, 512, False),
    (32, 2, 48, 256, 512, True),
    (6, 1, 3, 1024, 2048, False),
    (4, 4, 4, 8192, 192, False),
    (2, 2, 3, 16384, 64, False),
    # down with 2 and 4 positions per lane, more than one token per expert
    (3, 4, 4, 256, 4096, True),
    (5, 3, 3, 128, 8192, True),
    # gate/up with 4 positions per lane on a ragged row (H = 7168: 224 of 256)
    (4, 8, 16, 7168, 256, False),
    # the most pairs the union path takes (L * k = 1024): 32 tokens x 32 experts each
    # (matrix-core tiles: every expert serves about 16 tokens), and 16 x 64 on the GEMV units
    (32, 32, 64, 512, 256, False),
    (16, 64, 96, 256, 128, False),
    # the largest expert count (E = 16384)
    (8, 8, 16384, 64, 64, False),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "L%d_k%d_E%d_H%d_I%d_dup%d" % s)
def test_small_shapes(shape):
    L, k, E, H, I, dup = shape
    x, ids, tw, bank = synth.random_problem(L, k, E, H, I, seed=sum(shape), dup=dup)
    check_layer(x, ids, tw, bank, "small")


def test_all_tokens_same_expert_and_heavy_expert():
    # one expert serves every token (more tokens than one register chunk)
    E, H, I = 4, 1024, 256
    for L in (5, 13, 32):
        x, _, tw, bank = synth.random_problem(L, 2, E, H, I, seed=L)
        ids = np.tile(np.array([[1, 3]], np.int32), (L, 1))
        check_layer(x, ids, tw, bank, "same-expert L=%d" % L)


def test_bf16_output_is_rne_of_fp32_output():
    x, ids, tw, bank = synth.random_problem(4, 4, 9, 2048, 512, seed=3)
    say("bf16 vs fp32 output")
    o32, _ = run_layer(x, ids, tw, bank, torch.float32)
    o16, _ = run_layer(x, ids, tw, bank, torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))


def test_stages_split_equals_forward_and_determinism():
    x, ids, tw, bank = synth.random_problem(6, 4, 20, 2048, 512, seed=4)
    say("stages split / determinism")
    a, _ = run_layer(x, ids, tw, bank)
    b, _ = run_layer(x, ids, tw, bank, stages_split=True)
    c, _ = run_layer(x, ids, tw, bank)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


def test_workspace_reuse_across_shapes():
    # one workspace (sized for the largest call) reused by calls of other shapes
    q = _q()
    big = synth.random_problem(8, 8, 32, 2048, 512, seed=5)
    small = synth.random_problem(2, 8, 32, 2048, 512, seed=6)
    ws = q.new_workspace(8, 8, 32, 2048, 512)
    say("workspace reuse")
    for (x, ids, tw, bank) in (big, small, big):
        ref = oracle.forward_pairs(x, ids, tw, bank)
        out = q.forward_bank(x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), bank.to("cuda"),
                             out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH


def test_garbage_workspace_and_repeated_calls():
    # a workspace holding garbage needs no set-up; repeated calls and
    # repeated stage-only calls on it all give the oracle's result
    q = _q()
    x, ids, tw, bank = synth.random_problem(4, 8, 64, 1024, 256, seed=13)
    ref = oracle.forward_pairs(x, ids, tw, bank)
    xd, idd, twd, bk = x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), bank.to("cuda")
    n = q.moe_swiglu_q4_workspace_bytes(4, 8, 64, 1024, 256)
    ws = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    say("garbage workspace")
    outs = []
    for _ in range(3):
        outs.append(q.forward_bank(xd, idd, twd, bk, out_dtype=torch.float32, workspace=ws))
    out = torch.empty((4, 1024), dtype=torch.float32, device="cuda")
    for st in (q.MOE_Q4_STAGE_GATEUP, q.MOE_Q4_STAGE_GATEUP, q.MOE_Q4_STAGE_DOWN, q.MOE_Q4_STAGE_DOWN):
        q.forward_bank(xd, idd, twd, bk, out=out, out_dtype=torch.float32, workspace=ws, stages=st)
    outs.append(out)
    torch.cuda.synchronize()
    assert rel_err_rows(outs[0].cpu().numpy(), ref).max() <= ARITH
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_invalid_ids_set_status_and_drop_routes():
    q = _q()
    x, ids, tw, bank = synth.random_problem(3, 2, 6, 256, 128, seed=7)
    bad = ids.copy()
    bad[1, 1] = 6
    bad[2, 0] = -3
    say("invalid ids")
    out, ws = run_layer(x, bad, tw, bank)
    status, _ = q.moe_q4_read_device_status(ws)
    assert status & q.MOE_Q4_DEV_BAD_ID
    # expected: the same layer with the invalid routes' weights set to zero
    keep = ids.copy()
    keep[1, 1] = 0
    keep[2, 0] = 0
    tw0 = tw.copy()
    tw0[1, 1] = 0
    tw0[2, 0] = 0
    ref = oracle.forward_pairs(x, keep, tw0, bank)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH
    q.moe_q4_clear_device_status(ws)
    torch.cuda.synchronize()
    assert q.moe_q4_read_device_status(ws)[0] == 0


def test_all_ids_invalid_gives_zero_output():
    x, ids, tw, bank = synth.random_problem(2, 2, 4, 256, 128, seed=8)
    say("all ids invalid")
    out, _ = run_layer(x, np.full_like(ids, 99), tw, bank, torch.bfloat16)
    assert (out.float() == 0).all()


# ---------------------------------------------------------------------------
# the workload shapes at full size (every output checked)
# ---------------------------------------------------------------------------

FULL = [
    ("verify", 1, 0), ("verify", 2, 40), ("verify", 3, 60), ("verify", 4, 74), ("verify", 8, 7),
    ("flash", 1, 0), ("flash", 4, 41),
    ("small", 8, 0), ("small", 16, 3), ("small", 32, 15),
    ("small_pooled", 8, 0), ("small_pooled", 16, 5), ("small_pooled", 32, 9),
]


@pytest.mark.parametrize("wl,L,layer", FULL, ids=lambda v: str(v))
def test_full_size_layers(wl, L, layer):
    w = synth.WORKLOADS[wl]
    say("full", w.name, "L", L, "layer", layer)
    lay = synth.make_layer(w, L, layer, seed=0, device="cuda")
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, w.name)


def test_full_bank_layer_id_range():
    # one layer with the whole E=256 bank resident (ids span the full range)
    w = synth.WORKLOADS["verify"]
    say("full bank E=256 H=6144 I=2048 L=2")
    lay = synth.make_layer(w, 2, 11, seed=0, device="cuda", compact=False)
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, "full-bank")


@pytest.mark.parametrize("L", [1, 4])
def test_deepseek_shaped_layer_full_size(L):
    # E=256 top-8, hidden 7168, expert intermediate 2048 (four positions per
    # lane on a row of 224), independent uniform routes, every output checked
    w = synth.Workload("deepseek_shape_E256_k8_H7168_I2048", 256, 8, 7168, 2048, (1, 4), "uniform", 4)
    say("full", w.name, "L", L)
    lay = synth.make_layer(w, L, 1, seed=0, device="cuda")
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, w.name)


# ---------------------------------------------------------------------------
# tiny, zero and saturated activations (every codec)
# ---------------------------------------------------------------------------

def _check_tiny(x, ids, tw, bank, label):
    q = _q()
    say(label, bank.codec, "L=%d k=%d E=%d H=%d I=%d" % (ids.shape[0], ids.shape[1], bank.E, x.shape[1],
                                                         bank.wg.shape[1]))
    ref = oracle.forward_pairs_q(bank.codec, x.cpu(), ids, tw, bank.to("cpu"))
    dev = torch.device("cuda")
    bk = bank.to(dev)
    out = q.forward_bank_codec(x.to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev), bk,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    err = rel_err_rows(got, ref)
    print(f"  row rel errs {err}; |ref| row maxima {np.abs(ref).max(axis=1)}", flush=True)
    assert np.isfinite(got).all()
    assert np.abs(ref[0]).max() < 1e-30 and np.abs(ref[3]).max() < 1e-30  # the regime the case is about
    assert (got[1] == 0).all() and (ref[1] == 0).all()
    assert err.max() <= ARITH


@pytest.mark.parametrize("codec", ALL_CODECS)
def test_tiny_and_zero_activations(codec):
    H, I = (512, 256)
    x, ids, tw, bank = synth.random_problem_q(codec, 5, 4, 8, H, I, seed=31)
    x, ids, tw = tiny_zero_saturated(x, ids, tw, bank, e_star=5)
    _check_tiny(x, ids, tw, bank, "tiny/zero/saturated small")


@pytest.mark.parametrize("codec", ALL_CODECS)
def test_tiny_and_zero_activations_full_size(codec):
    # one GLM-5.2-style verify layer (E=256 top-8, H=6144, I=2048) at L=4
    w = synth.WORKLOADS["verify"]
    lay = synth.make_layer_q(codec, w, 4, 30, seed=0, device="cuda")
    x, ids, tw = tiny_zero_saturated(lay.x, lay.ids, lay.weights, lay.bank, e_star=int(lay.ids[2, 1]))
    _check_tiny(x, ids, tw, lay.bank, "tiny/zero/saturated full-size verify")


# ---------------------------------------------------------------------------
# matrix-core tiles (more than 8 tokens; experts with at least 4 tokens when
# such experts are at least half of the distinct ones)
# ---------------------------------------------------------------------------

def _pooled_ids(rng, L, k, pool, E):
    """Each token takes its k experts from a shared pool of `pool` ids."""
    members = rng.permutation(E)[:pool]
    return np.stack([rng.permutation(members)[:k] for _ in range(L)]).astype(np.int32)


def test_matrix_core_tile_token_counts():
    # one expert per token count around the 16-token blocks of a tile:
    # 32, 17, 16 and 15 tokens (every expert has at least 4)
    E, H, I, L = 8, 512, 256, 32
    x, _, tw, bank = synth.random_problem(L, 3, E, H, I, seed=91)
    t = np.arange(L)
    ids = np.stack([np.full(L, 2), np.where(t < 17, 0, 5), np.where(t >= 16, 1, 6)], axis=1).astype(np.int32)
    check_layer(x, ids, tw, bank, "tile token counts 32/17/16/15")


@pytest.mark.parametrize("L,k,pool,E,H,I", [(16, 4, 8, 32, 512, 256), (32, 8, 12, 64, 256, 512),
                                            (12, 2, 4, 16, 768, 768), (24, 6, 16, 64, 2048, 512)])
def test_matrix_core_pooled_routes(L, k, pool, E, H, I):
    rng = np.random.default_rng(1000 + L + pool)
    x, _, tw, bank = synth.random_problem(L, k, E, H, I, seed=L * pool)
    ids = _pooled_ids(rng, L, k, pool, E)
    check_layer(x, ids, tw, bank, "pooled pool=%d" % pool)


def test_matrix_core_tiles_beside_gemv_experts():
    # 8 hot experts with 9 tokens each run as tiles; the cold experts (1 to
    # 5 tokens) of the same call run on the GEMV units
    rng = np.random.default_rng(77)
    E, H, I, L = 32, 1024, 512, 24
    x, _, tw, bank = synth.random_problem(L, 4, E, H, I, seed=77)
    hot = np.arange(8)
    ids = np.stack([np.concatenate([rng.permutation(hot)[:3], rng.integers(8, 16, size=1)]) for _ in range(L)])
    ids = ids.astype(np.int32)
    n = np.bincount(ids.ravel(), minlength=E)
    assert (n[:8] >= 4).all() and (n[8:16] < 4).any()
    check_layer(x, ids, tw, bank, "tiles beside GEMV experts")


def test_matrix_core_unaligned_scales_take_gemv_units():
    # scale arrays 4 but not 8 bytes aligned: the launch keeps the GEMV
    # kernels (the tiles read 8-byte scale pieces)
    rng = np.random.default_rng(5)
    E, H, I, L = 16, 512, 256, 16
    x, _, tw, bank = synth.random_problem(L, 4, E, H, I, seed=5)
    ids = _pooled_ids(rng, L, 4, 8, E)

    def shifted(t):  # a device view 4 bytes past an 8-byte boundary (the binding keeps device tensors as they are)
        flat = torch.empty(t.numel() + 2, dtype=t.dtype, device="cuda")
        view = flat[2:].view(t.shape)
        view.copy_(t.to("cuda"))
        assert view.data_ptr() % 8 == 4
        return view

    gpu = bank.to("cuda")
    unaligned = dataclasses.replace(gpu, sg=shifted(bank.sg), bg=shifted(bank.bg), su=shifted(bank.su),
                                    bu=shifted(bank.bu), sd=shifted(bank.sd), bd=shifted(bank.bd))
    got, ref = check_layer(x, ids, tw, unaligned, "unaligned scales")
    aligned, _ = check_layer(x, ids, tw, bank, "aligned scales")
    assert np.abs(got - aligned).max() <= 1e-3 * np.abs(ref).max()
