"""GPU parity of the sorted (MFMA) path over mxfp4 banks (needs an MI355X).

Inputs longer than one union launch (more than 32 tokens) with H and I
multiples of 256 take the sorted path: pairs sorted by expert, gate/up and
down as grouped bf16 MFMA GEMMs.  The E8M0 block scale 2^(e - 127) is folded
into gfx950's scaled E2M1 -> bf16 conversion, which is exact while every
E2M1 magnitude times the scale is a normal bf16 (2 <= e <= 252), so the
matrix cores accumulate over the whole reduction with no per-group fp32
work.  Blocks holding any other exponent byte are recomputed by an exact
pass: one MFMA chain per 32-input block and the scale applied in fp32
(subnormal scales, NaN for e = 255), as in the oracle.

Bars: fp32 outputs within a per-row normwise relative error of 1e-3 (the
contract) and 2e-4 (the arithmetic: exact products, fp32 accumulation, h as
a bf16 hi + lo pair of 16 significant bits); bf16 outputs the
round-to-nearest-even of the fp32 outputs, bit for bit.  The format is the
GLM-5.2 bank format of the mlx discussion "Small-L fused expert gather for
fine-grained MoE decode" (section "The data"); bit layouts from the OCP MX
v1.0 specification.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tile_sampling import coverage_tokens

pytestmark = pytest.mark.gpu

CONTRACT = 1e-3
ARITH = 2e-4


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
    H, I = x.shape[1], bk.wg.shape[1]
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


def check_path(ws):
    q = _q()
    status, path = q.moe_q4_read_device_status(ws)
    assert status == 0 and path == q.MOE_Q4_PATH_SORTED


def check_layer(x, ids, tw, bank, label):
    say(label, "mxfp4 sorted T=%d k=%d E=%d H=%d I=%d" % (ids.shape[0], ids.shape[1], bank.E, x.shape[1],
                                                          bank.wg.shape[1]))
    ref = oracle.forward_pairs_mx(x.cpu(), ids, tw, bank.to("cpu"))
    out, ws = run_layer(x, ids, tw, bank)
    got = out.float().cpu().numpy()
    err = rel_err_rows(got, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= CONTRACT
    assert err.max() <= ARITH
    check_path(ws)
    return got, ref


# (T, k, E, H, I, dup): mean pairs per expert T*k/E selects 1, 2, 3 or 4
# 32-row blocks per tile; ragged last tiles; duplicate ids within a token
SMALL = [
    (33, 8, 64, 1024, 1024, False),   # first T past the union path, ~4 pairs per expert
    (40, 4, 8, 1024, 1024, False),    # 20 per expert -> 1 block
    (80, 4, 8, 1024, 2048, False),    # 40 -> 2 blocks
    (121, 4, 8, 2048, 1024, False),   # ~60 -> 3 blocks
    (203, 4, 8, 1024, 1024, False),   # ~100 -> 4 blocks, experts over several tiles
    (64, 8, 16, 1024, 1024, True),    # duplicate ids
    (300, 2, 4, 1024, 1024, False),   # 150 per expert
    # widths that are multiples of 256, not of 1024 (one iteration at 256)
    (40, 4, 8, 1280, 768, False),
    (121, 4, 8, 768, 256, False),
    (203, 4, 8, 256, 1280, False),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T%d_k%d_E%d_H%d_I%d%s" % (*s[:5], "_dup" if s[5] else ""))
def test_mx_sorted_small(shape):
    T, k, E, H, I, dup = shape
    assert _q().moe_swiglu_codec_workspace_bytes(_q().MOE_Q4_CODEC_MXFP4, T, k, E, H, I) > 0
    x, ids, tw, bank = synth.random_problem_mx(T, k, E, H, I, seed=sum(shape), dup=dup)
    check_layer(x, ids, tw, bank, "small")


def test_mx_sorted_bf16_rne_stages_split_and_determinism():
    x, ids, tw, bank = synth.random_problem_mx(90, 4, 8, 1024, 1024, seed=5)
    say("mxfp4 sorted bf16 / stages / determinism")
    o32, ws = run_layer(x, ids, tw, bank, torch.float32)
    check_path(ws)
    o16, _ = run_layer(x, ids, tw, bank, torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    osp, _ = run_layer(x, ids, tw, bank, torch.float32, stages_split=True)
    assert torch.equal(o32.view(torch.int32), osp.view(torch.int32))
    again, _ = run_layer(x, ids, tw, bank, torch.float32)
    assert torch.equal(o32.view(torch.int32), again.view(torch.int32))


def test_mx_sorted_matches_token_chunks_on_unaligned_scales():
    # scale arrays that are not 8-byte aligned run as union token chunks;
    # both paths agree with the oracle
    q = _q()
    T, k, E, H, I = 48, 4, 8, 1024, 1024
    x, ids, tw, bank = synth.random_problem_mx(T, k, E, H, I, seed=8)
    ref = oracle.forward_pairs_mx(x, ids, tw, bank)
    bk = bank.to("cuda")
    xd, idd, twd = x.cuda(), torch.from_numpy(ids).cuda(), torch.from_numpy(tw).cuda()
    n = q.moe_swiglu_mxfp4_workspace_bytes(T, k, E, H, I)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    say("mxfp4 sorted vs chunks")
    a = q.moe_swiglu_mxfp4_forward(xd, idd, twd, *bk.tensors(), out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert q.moe_q4_read_device_status(ws)[1] == q.MOE_Q4_PATH_SORTED
    shifted = []
    for t in bk.tensors():
        if t.dtype == torch.uint8:  # the E8M0 arrays, one byte past an aligned start
            buf = torch.empty(t.numel() + 16, dtype=torch.uint8, device="cuda")
            v = buf[1:1 + t.numel()].view(t.shape)
            v.copy_(t)
            shifted.append(v)
        else:
            shifted.append(t)
    b = q.moe_swiglu_mxfp4_forward(xd, idd, twd, *shifted, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert q.moe_q4_read_device_status(ws)[1] == q.MOE_Q4_PATH_UNION
    assert rel_err_rows(a.cpu().numpy(), ref).max() <= ARITH
    assert rel_err_rows(b.cpu().numpy(), ref).max() <= 6e-4  # the union path's bound


def test_mx_sorted_invalid_ids_dropped_and_reported():
    q = _q()
    x, ids, tw, bank = synth.random_problem_mx(70, 4, 8, 1024, 1024, seed=9)
    ids = ids.copy()
    ids[3, 1] = -1
    ids[50, 0] = 8
    bad = (ids < 0) | (ids >= 8)
    say("mxfp4 sorted invalid ids")
    ref = oracle.forward_pairs_mx(x, np.where(bad, 0, ids), np.where(bad, 0.0, tw).astype(np.float32), bank)
    out, ws = run_layer(x, ids, tw, bank)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= ARITH
    status, path = q.moe_q4_read_device_status(ws)
    assert status == q.MOE_Q4_DEV_BAD_ID and path == q.MOE_Q4_PATH_SORTED


def _extreme_bank(T, E, H, I, seed):
    """k = 1 routes.  Expert 1 carries exponent bytes outside the folded
    range (gate 0 and 1: subnormal and 2^-126 block scales; down rows 5 and
    77: 253 and 254), balanced by large up and down scales so that its
    outputs stay normal fp32 values; its down row 300 (another column block)
    holds 252.  Expert 2 sits on the edges of the folded range: every gate
    byte 2, every up byte 240."""
    x, ids, tw, bank = synth.random_problem_mx(T, 1, E, H, I, seed=seed)
    rng = np.random.default_rng(seed)
    sg, su, sd = bank.sg.clone(), bank.su.clone(), bank.sd.clone()
    sg[1] = torch.from_numpy(rng.integers(0, 2, size=tuple(sg[1].shape)).astype(np.uint8))
    su[1] = 200
    sd[1] = 180
    sd[1, 5] = 253
    sd[1, 77] = 254
    sd[1, 300] = 252
    sg[2] = 2
    su[2] = 240
    bank = type(bank)(bank.wg, sg, bank.wu, su, bank.wd, sd)
    return x, ids, tw, bank


def test_mx_sorted_exact_pass_for_scales_outside_the_folded_range():
    T, E, H, I = 96, 4, 1024, 1024
    x, ids, tw, bank = _extreme_bank(T, E, H, I, seed=13)
    say("mxfp4 sorted extreme scales")
    ref = oracle.forward_pairs_mx(x, ids, tw, bank)
    out, ws = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    assert np.array_equal(np.isfinite(got), np.isfinite(ref))
    fin = np.isfinite(ref).all(axis=1)
    err = rel_err_rows(got[fin], ref[fin])
    print(f"  max row rel err {err.max():.3e} over {fin.sum()} finite rows", flush=True)
    assert err.max() <= ARITH
    check_path(ws)


def test_mx_sorted_nan_scale_reaches_exactly_its_outputs():
    # gate scale 255 on one row of expert 1 makes h of its pairs NaN (every
    # output of the tokens routed to it); down scale 255 on row 19 of expert
    # 2 makes column 19 NaN for the tokens routed to expert 2
    T, k, E, H, I = 64, 2, 5, 1024, 1024
    x, ids, tw, bank = synth.random_problem_mx(T, k, E, H, I, seed=9)
    bank.sg[1, 7, 3] = 255
    bank.sd[2, 19, 1] = 255
    say("mxfp4 sorted NaN scales")
    ref = oracle.forward_pairs_mx(x, ids, tw, bank)
    out, _ = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.isfinite(got[fin]).all()
    assert np.max(np.abs(got[fin] - ref[fin])) <= ARITH * np.max(np.abs(ref[fin]))


# ---------------------------------------------------------------------------
# the prefill workload (E = 256, top-8, H = 4096, I = 2048) in mxfp4 at full
# size, and the long-prefill regime (T = 16384, 4 row blocks per tile):
# sampled tokens against the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [512, 2048, 16384])
def test_mx_sorted_prefill_full_size_sampled(T):
    w = synth.WORKLOADS["prefill"]
    lay = synth.make_layer_mx(w, T, 0, seed=0, device="cuda")
    say("mxfp4 prefill", T, "u", lay.bank.E)
    out, ws = run_layer(lay.x, lay.ids, lay.weights, lay.bank)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    check_path(ws)
    sample = coverage_tokens(lay.ids, lay.bank.E, n=64, seed=T)
    used = np.unique(lay.ids[sample])
    sub = lay.bank.select(used).to("cpu")
    ref = oracle.forward_pairs_mx(lay.x[sample].cpu(), np.searchsorted(used, lay.ids[sample]).astype(np.int32),
                                  lay.weights[sample], sub)
    err = rel_err_rows(got[sample], ref)
    print(f"  sampled rows {sample}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= ARITH
