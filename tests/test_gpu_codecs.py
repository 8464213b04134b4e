"""GPU parity of the union path over the further weight codecs (needs an MI355X).

Codecs: 4-bit affine with group 32, nvfp4 (E2M1 elements, an FP8 E4M3 scale
per 16 inputs), mxfp4, 8-bit affine with group 64 and mxfp8 (E4M3 elements,
an E8M0 scale per 32 inputs) through the generic codec entry point, each
against the CPU oracle's evaluation of the same codec.  The pages name these storage
modes (the dequant-mode comparison of the mlx discussion "Small-L fused
expert gather for fine-grained MoE decode"; nvfp4 among the quantized modes
of PR 4572 on the page "MoE GatherQMM small-M verify cost", Facts) without
bit layouts; the layouts are the OCP ones (include/moe_q4.h).

Bars as for the 4-bit affine banks: fp32 outputs within a per-row normwise
relative error of 1e-3 (the contract) and 6e-4 (the arithmetic: exact
element products accumulated in fp32 for gate and up, h rounded to fp16
after an exact power-of-two rescale for down); bf16 outputs the
round-to-nearest-even of the fp32 outputs.
"""

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

CONTRACT = 1e-3
ARITH = 6e-4
CODECS = ["affine4_g32", "nvfp4", "mxfp4", "affine8_g64", "mxfp8"]


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
        n = q.moe_swiglu_codec_workspace_bytes(q.CODECS[bank.codec][0], L, k, bk.E, H, I)
        assert n > 0
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    if stages_split:
        out = torch.empty((L, H), dtype=out_dtype, device=dev)
        for st in (q.MOE_Q4_STAGE_GATEUP, q.MOE_Q4_STAGE_DOWN):
            q.forward_bank_codec(xd, idd, twd, bk, out=out, out_dtype=out_dtype, workspace=ws, stages=st)
    else:
        out = q.forward_bank_codec(xd, idd, twd, bk, out_dtype=out_dtype, workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def check_layer(x, ids, tw, bank, label):
    say(label, bank.codec, "L=%d k=%d E=%d H=%d I=%d" % (ids.shape[0], ids.shape[1], bank.E, x.shape[1],
                                                         bank.wg.shape[1]))
    ref = oracle.forward_pairs_q(bank.codec, x.cpu(), ids, tw, bank.to("cpu"))
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
    # (L, k, E, H, I, dup): odd H/32 and I/32, ragged lane groups, several
    # positions per lane, duplicates, one and many tokens
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
    (3, 4, 4, 256, 4096, True),
    (4, 8, 16, 7168, 256, False),
    (32, 32, 64, 512, 256, False),   # the union path's pair limit, L * k = 1024
]


# the same cases with H and I multiples of 64 (group-64 8-bit affine codes)
SMALL_SHAPES_64 = [
    (1, 2, 4, 64, 64, False),
    (2, 2, 4, 128, 256, False),
    (3, 2, 6, 384, 192, True),
    (5, 3, 7, 320, 128, True),
    (8, 4, 16, 2048, 256, False),
    (4, 8, 12, 4096, 192, True),
    (2, 8, 64, 6144, 128, False),
    (16, 4, 40, 512, 512, False),
    (32, 2, 48, 256, 512, True),
    (6, 1, 3, 1088, 2048, False),
    (4, 4, 4, 8192, 192, False),
    (3, 4, 4, 256, 4096, True),
    (4, 8, 16, 7168, 256, False),
    (32, 32, 64, 512, 256, False),
]
SHAPE_CASES = [(c, sh) for c in CODECS for sh in (SMALL_SHAPES_64 if c == "affine8_g64" else SMALL_SHAPES)]


@pytest.mark.parametrize("codec,shape", SHAPE_CASES,
                         ids=[f"{c}-L%d_k%d_E%d_H%d_I%d_dup%d" % sh for c, sh in SHAPE_CASES])
def test_codec_small_shapes(codec, shape):
    L, k, E, H, I, dup = shape
    x, ids, tw, bank = synth.random_problem_q(codec, L, k, E, H, I, seed=sum(shape), dup=dup)
    check_layer(x, ids, tw, bank, "small")


@pytest.mark.parametrize("codec", CODECS)
def test_codec_bf16_rne_stage_split_and_determinism(codec):
    x, ids, tw, bank = synth.random_problem_q(codec, 6, 4, 20, 2048, 512, seed=4)
    say(codec, "bf16 / stage split / determinism")
    a, _ = run_layer(x, ids, tw, bank)
    b, _ = run_layer(x, ids, tw, bank, stages_split=True)
    c, _ = run_layer(x, ids, tw, bank)
    o16, _ = run_layer(x, ids, tw, bank, torch.bfloat16)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))
    assert torch.equal(a.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))


@pytest.mark.parametrize("codec", CODECS)
def test_codec_invalid_ids_set_status_and_drop_routes(codec):
    q = _q()
    x, ids, tw, bank = synth.random_problem_q(codec, 3, 2, 6, 256, 128, seed=7)
    bad = ids.copy()
    bad[1, 1] = 6
    bad[2, 0] = -3
    say(codec, "invalid ids")
    out, ws = run_layer(x, bad, tw, bank)
    assert q.moe_q4_read_device_status(ws)[0] & q.MOE_Q4_DEV_BAD_ID
    keep, tw0 = ids.copy(), tw.copy()
    for t, j in ((1, 1), (2, 0)):
        keep[t, j], tw0[t, j] = 0, 0
    ref = oracle.forward_pairs_q(codec, x, keep, tw0, bank)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH


def test_nvfp4_nan_scale_reaches_exactly_its_outputs():
    # an E4M3 NaN scale (0x7F) on gate row 7 of expert 1 makes h of its pairs
    # NaN; on down row 19 of expert 2, column 19 of the tokens routed to it
    L, k, E, H, I = 4, 2, 5, 256, 128
    x, _, tw, bank = synth.random_problem_q("nvfp4", L, k, E, H, I, seed=9)
    ids = np.array([[1, 0], [2, 3], [0, 4], [3, 2]], np.int32)
    bank.sg[1, 7, 5] = 0x7F
    bank.sd[2, 19, 3] = 0xFF
    say("nvfp4 NaN scales")
    ref = oracle.forward_pairs_q("nvfp4", x, ids, tw, bank)
    out, _ = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[0]).all() and np.isnan(got[1, 19]) and np.isnan(got[3, 19])
    fin = ~np.isnan(ref)
    assert np.max(np.abs(got[fin] - ref[fin])) <= ARITH * np.max(np.abs(ref[fin]))


def test_nvfp4_subnormal_and_extreme_scales():
    # E4M3 scales across the whole range: subnormals (codes 1..7), the
    # largest (0x7E = 448) and zero, mixed inside every row
    x, ids, tw, bank = synth.random_problem_q("nvfp4", 4, 4, 8, 512, 256, seed=12)
    g = torch.Generator().manual_seed(3)
    for t in (bank.sg, bank.su, bank.sd):
        codes = torch.randint(0, 0x7F, t.shape, generator=g, dtype=torch.int64)  # every finite positive code
        t.copy_(codes.to(torch.uint8))
    check_layer(x, ids, tw, bank, "all E4M3 scales")


@pytest.mark.parametrize("codec", CODECS)
@pytest.mark.parametrize("L,layer", [(1, 0), (8, 7)], ids=lambda v: str(v))
def test_codec_full_size_verify_layers(codec, L, layer):
    w = synth.WORKLOADS["verify"]
    say("full", w.name, codec, "L", L, "layer", layer)
    lay = synth.make_layer_q(codec, w, L, layer, seed=0, device="cuda")
    check_layer(lay.x, lay.ids, lay.weights, lay.bank, w.name)


@pytest.mark.parametrize("codec", CODECS)
def test_codec_long_inputs_run_as_token_chunks(codec):
    # 70 tokens at top-8: chunks of 32, 32 and 6 tokens on one workspace;
    # an invalid id in the last chunk must reach the call's status word
    # (I = 320 is not a multiple of 256, so mxfp4 stays on token chunks too)
    q = _q()
    L, k, E, H, I = 70, 8, 64, 512, 320
    x, ids, tw, bank = synth.random_problem_q(codec, L, k, E, H, I, seed=21)
    say(codec, "token chunks L=70")
    ref = oracle.forward_pairs_q(codec, x, ids, tw, bank)
    out, ws = run_layer(x, ids, tw, bank)
    assert q.moe_swiglu_codec_workspace_bytes(q.CODECS[codec][0], L, k, E, H, I) == \
        q.moe_swiglu_codec_workspace_bytes(q.CODECS[codec][0], 32, k, E, H, I)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH
    assert q.moe_q4_read_device_status(ws)[0] == 0
    bad = ids.copy()
    bad[66, 3] = E + 5
    out2, ws2 = run_layer(x, bad, tw, bank)
    assert q.moe_q4_read_device_status(ws2)[0] & q.MOE_Q4_DEV_BAD_ID
    keep, tw0 = ids.copy(), tw.copy()
    keep[66, 3], tw0[66, 3] = 0, 0
    assert rel_err_rows(out2.cpu().numpy(), oracle.forward_pairs_q(codec, x, keep, tw0, bank)).max() <= ARITH


@pytest.mark.parametrize("codec", CODECS)
def test_codec_wide_hidden_runs_smaller_chunks(codec):
    # H = 4096: 32 tokens' activations do not fit one workgroup's LDS, so the
    # chunks hold fewer tokens (mxfp4 stays on the union path: I = 320 is not
    # a multiple of 256)
    q = _q()
    L, k, E, H, I = 40, 8, 16, 4096, 320
    x, ids, tw, bank = synth.random_problem_q(codec, L, k, E, H, I, seed=23)
    say(codec, "wide hidden L=40 H=4096")
    ref = oracle.forward_pairs_q(codec, x, ids, tw, bank)
    out, ws = run_layer(x, ids, tw, bank)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH
    assert q.moe_q4_read_device_status(ws) == (0, q.MOE_Q4_PATH_UNION)


def test_codec_entry_for_affine_group64_is_the_q4_forward():
    q = _q()
    x, ids, tw, bank = synth.random_problem(4, 4, 9, 1024, 512, seed=14)
    say("codec 0 == moe_swiglu_q4_forward")
    xd, idd, twd, bk = x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda(), bank.to("cuda")
    a = q.forward_bank(xd, idd, twd, bk, out_dtype=torch.float32)
    b = q.moe_swiglu_codec_forward("affine4_g64", xd, idd, twd, *bk.tensors(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
