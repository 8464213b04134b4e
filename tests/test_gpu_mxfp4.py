"""GPU parity of the mxfp4 union path against the CPU oracle (needs an MI355X).

mxfp4 gs32 banks: FP4 E2M1 elements with one E8M0 scale byte per 32 inputs
(the format of the GLM-5.2 banks on the mlx discussion page "Small-L fused
expert gather for fine-grained MoE decode", section "The data"; bit layouts
from the OCP MX v1.0 specification).

Bars as for the affine banks: fp32 layer outputs within a per-row normwise
relative error of 1e-3 (the contract) and of 6e-4, the bound the arithmetic
gives.  Gate and up multiply E2M1 values (exact in bf16) by bf16 activations
into fp32 and apply the power-of-two scale exactly, so they err by fp32
accumulation only; the down projection reads h rounded to fp16 after an
exact power-of-two rescale (unit roundoff 2^-11, about 2.8e-4 normwise with
random-sign rounding errors).  bf16 outputs equal the round-to-nearest-even
of the fp32 outputs bit for bit.  A NaN scale byte (255) makes every output
that its block reaches NaN, as in the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

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


def run_layer(x, ids, tw, bank, out_dtype=torch.float32, stages_split=False, workspace=None):
    q = _q()
    dev = torch.device("cuda")
    xd = x.to(dev)
    idd = torch.as_tensor(np.asarray(ids, np.int32)).to(dev)
    twd = torch.as_tensor(np.asarray(tw, np.float32)).to(dev)
    bk = bank.to(dev)
    L, k = idd.shape
    H, I = x.shape[1], bk.wg.shape[1]
    ws = workspace
    if ws is None:
        n = q.moe_swiglu_mxfp4_workspace_bytes(L, k, bk.E, H, I)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    if stages_split:
        out = torch.empty((L, H), dtype=out_dtype, device=dev)
        q.forward_bank_mx(xd, idd, twd, bk, out=out, out_dtype=out_dtype, workspace=ws, stages=q.MOE_Q4_STAGE_GATEUP)
        q.forward_bank_mx(xd, idd, twd, bk, out=out, out_dtype=out_dtype, workspace=ws, stages=q.MOE_Q4_STAGE_DOWN)
    else:
        out = q.forward_bank_mx(xd, idd, twd, bk, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def check_layer(x, ids, tw, bank, label):
    say(label, "mxfp4 L=%d k=%d E=%d H=%d I=%d" % (ids.shape[0], ids.shape[1], bank.E, x.shape[1],
                                                   bank.wg.shape[1]))
    ref = oracle.forward_pairs_mx(x.cpu(), ids, tw, bank.to("cpu"))
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


SMALL_SHAPES = [
    # (L, k, E, H, I, dup): H/32 and I/32 odd (only the mxfp4 banks allow
    # multiples of 32 that are not multiples of 64), ragged lane groups,
    # several positions per lane, duplicates, one and many tokens
    (1, 2, 4, 64, 64, False),
    (2, 2, 4, 96, 256, False),
    (3, 2, 6, 352, 224, True),
    (5, 3, 7, 160, 288, True),
    (8, 4, 16, 2048, 256, False),
    (4, 8, 12, 4096, 160, True),
    (2, 8, 64, 6144, 128, False),
    (16, 4, 40, 512, 512, False),
    (32, 2, 48, 256, 480, True),
    (6, 1, 3, 1056, 2048, False),
    (4, 4, 4, 8192, 192, False),
    (2, 2, 3, 16384, 64, False),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "L%d_k%d_E%d_H%d_I%d_dup%d" % s)
def test_mx_small_shapes(shape):
    L, k, E, H, I, dup = shape
    x, ids, tw, bank = synth.random_problem_mx(L, k, E, H, I, seed=sum(shape), dup=dup)
    check_layer(x, ids, tw, bank, "small")


def test_mx_bf16_output_is_rne_of_fp32_output():
    x, ids, tw, bank = synth.random_problem_mx(4, 4, 9, 2048, 512, seed=3)
    say("mxfp4 bf16 vs fp32 output")
    o32, _ = run_layer(x, ids, tw, bank, torch.float32)
    o16, _ = run_layer(x, ids, tw, bank, torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))


def test_mx_stages_split_equals_forward_and_determinism():
    x, ids, tw, bank = synth.random_problem_mx(6, 4, 20, 2048, 512, seed=4)
    say("mxfp4 stages split / determinism")
    a, _ = run_layer(x, ids, tw, bank)
    b, _ = run_layer(x, ids, tw, bank, stages_split=True)
    c, _ = run_layer(x, ids, tw, bank)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


def test_mx_nan_scale_reaches_exactly_its_outputs():
    # gate scale 255 on one row of expert 1 makes h of its pairs NaN (so every
    # output of the tokens routed to expert 1); down scale 255 on row m of
    # expert 2 makes column m NaN for the tokens routed to expert 2
    L, k, E, H, I = 4, 2, 5, 256, 128
    x, ids, tw, bank = synth.random_problem_mx(L, k, E, H, I, seed=9)
    ids = np.array([[1, 0], [2, 3], [0, 4], [3, 2]], np.int32)
    bank.sg[1, 7, 3] = 255
    bank.sd[2, 19, 1] = 255
    say("mxfp4 NaN scales")
    ref = oracle.forward_pairs_mx(x, ids, tw, bank)
    out, _ = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[0]).all() and np.isnan(got[1, 19]) and np.isnan(got[3, 19])
    fin = ~np.isnan(ref)
    assert np.isfinite(got[fin]).all()
    assert np.max(np.abs(got[fin] - ref[fin])) <= ARITH * np.max(np.abs(ref[fin]))


def test_mx_invalid_ids_set_status_and_drop_routes():
    q = _q()
    x, ids, tw, bank = synth.random_problem_mx(3, 2, 6, 256, 128, seed=7)
    bad = ids.copy()
    bad[1, 1] = 6
    bad[2, 0] = -3
    say("mxfp4 invalid ids")
    out, ws = run_layer(x, bad, tw, bank)
    status, _ = q.moe_q4_read_device_status(ws)
    assert status & q.MOE_Q4_DEV_BAD_ID
    keep = ids.copy()
    keep[1, 1] = 0
    keep[2, 0] = 0
    tw0 = tw.copy()
    tw0[1, 1] = 0
    tw0[2, 0] = 0
    ref = oracle.forward_pairs_mx(x, keep, tw0, bank)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH


def test_mx_and_affine_calls_share_a_workspace():
    # calls over the two bank formats alternate on one workspace
    q = _q()
    L, k, E, H, I = 4, 4, 16, 1024, 256
    xm, idm, twm, bm = synth.random_problem_mx(L, k, E, H, I, seed=11)
    xa, ida, twa, ba = synth.random_problem(L, k, E, H, I, seed=11)
    n = max(q.moe_swiglu_mxfp4_workspace_bytes(L, k, E, H, I), q.moe_swiglu_q4_workspace_bytes(L, k, E, H, I))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("mxfp4 / affine alternate")
    rm = oracle.forward_pairs_mx(xm, idm, twm, bm)
    ra = oracle.forward_pairs(xa, ida, twa, ba)
    for _ in range(2):
        om, _ = run_layer(xm, idm, twm, bm, workspace=ws)
        oa = q.forward_bank(xa.cuda(), torch.from_numpy(ida).cuda(), torch.from_numpy(twa).cuda(), ba.to("cuda"),
                            out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert rel_err_rows(om.cpu().numpy(), rm).max() <= ARITH
        assert rel_err_rows(oa.cpu().numpy(), ra).max() <= ARITH


# ---------------------------------------------------------------------------
# the GLM-5.2 verify layer in mxfp4 at full size (every output checked)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,layer", [(1, 0), (2, 40), (4, 74), (8, 7)], ids=lambda v: str(v))
def test_mx_full_size_verify_layers(L, layer):
    w = synth.WORKLOADS["verify"]
    say("mxfp4 full", w.name, "L", L, "layer", layer)
    lay = synth.make_layer_mx(w, L, layer, seed=0, device="cuda")
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, w.name)


@pytest.mark.parametrize("L", [8, 32])
def test_mx_full_size_small_expert_layers(L):
    w = synth.WORKLOADS["small"]
    say("mxfp4 full", w.name, "L", L)
    lay = synth.make_layer_mx(w, L, 3, seed=0, device="cuda")
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, w.name)
