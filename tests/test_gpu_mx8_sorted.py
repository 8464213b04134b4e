"""GPU parity of the sorted (MFMA) path over mxfp8 banks (needs an MI355X).

mxfp8: FP8 E4M3 elements (one byte per input) with one E8M0 scale byte per
32 inputs (OCP MX v1.0; the mode of the dequant comparison on the mlx
discussion page "Small-L fused expert gather for fine-grained MoE decode").
Inputs longer than one union launch with H and I multiples of 256 take the
sorted path.  The scale 2^(e - 127) is folded into gfx950's scaled
E4M3 -> bf16 conversion, exact while every nonzero E4M3 magnitude (2^-9 to
448) times the scale is a normal bf16 (10 <= e <= 246); blocks holding
other exponent bytes are recomputed by the exact pass (per-32-input MFMA
chains, fp32 scaling), as for mxfp4.

Bars as for the other sorted paths: fp32 outputs within 1e-3 (the contract)
and 2e-4 (the arithmetic) normwise per row against the CPU oracle's mxfp8
evaluation; bf16 outputs the round-to-nearest-even of the fp32 outputs.
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
CODEC = "mxfp8"


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
    n = q.moe_swiglu_codec_workspace_bytes(q.CODECS[CODEC][0], L, k, bk.E, H, I)
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


def check_path(ws):
    q = _q()
    status, path = q.moe_q4_read_device_status(ws)
    assert status == 0 and path == q.MOE_Q4_PATH_SORTED


SMALL = [
    # (T, k, E, H, I, dup): 1, 2, 3 and 4 row blocks per tile, widths that are
    # multiples of 256 but not of 1024, duplicates
    (40, 4, 8, 1024, 1024, False),
    (80, 4, 8, 1024, 2048, False),
    (121, 4, 8, 2048, 768, False),
    (203, 4, 8, 1280, 1024, False),
    (64, 8, 16, 1024, 1024, True),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "T%d_k%d_E%d_H%d_I%d%s" % (*s[:5], "_dup" if s[5] else ""))
def test_mx8_sorted_small(shape):
    T, k, E, H, I, dup = shape
    x, ids, tw, bank = synth.random_problem_q(CODEC, T, k, E, H, I, seed=sum(shape), dup=dup)
    say("mxfp8 sorted", shape)
    ref = oracle.forward_pairs_q(CODEC, x, ids, tw, bank)
    out, ws = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    err = rel_err_rows(got, ref)
    print(f"  max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= CONTRACT and err.max() <= ARITH
    check_path(ws)


def test_mx8_sorted_bf16_rne_stages_split_and_determinism():
    x, ids, tw, bank = synth.random_problem_q(CODEC, 90, 4, 8, 1024, 1024, seed=5)
    say("mxfp8 sorted bf16 / stages / determinism")
    o32, ws = run_layer(x, ids, tw, bank, torch.float32)
    check_path(ws)
    o16, _ = run_layer(x, ids, tw, bank, torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    osp, _ = run_layer(x, ids, tw, bank, torch.float32, stages_split=True)
    assert torch.equal(o32.view(torch.int32), osp.view(torch.int32))
    again, _ = run_layer(x, ids, tw, bank, torch.float32)
    assert torch.equal(o32.view(torch.int32), again.view(torch.int32))


def test_mx8_sorted_exact_pass_and_nan_scales():
    # k = 1.  Expert 1: gate exponent bytes 3..9 (below the folded range),
    # balanced by large up and down scales, and down rows 5 and 77 at 247
    # and 250 (above it): the exact pass.  Expert 2: gate bytes 10, the
    # lower edge of the folded range, with up 200.  Expert 3: one NaN gate
    # scale byte, so every output of its tokens is NaN.
    T, E, H, I = 96, 4, 1024, 1024
    x, ids, tw, bank = synth.random_problem_q(CODEC, T, 1, E, H, I, seed=13)
    rng = np.random.default_rng(13)
    bank.sg[1] = torch.from_numpy(rng.integers(3, 10, size=tuple(bank.sg[1].shape)).astype(np.uint8))
    bank.su[1] = 200
    bank.sd[1] = 170
    bank.sd[1, 5] = 247
    bank.sd[1, 77] = 250
    bank.sg[2] = 10
    bank.su[2] = 200
    bank.sg[3, 7, 3] = 255
    say("mxfp8 sorted exact pass / NaN")
    ref = oracle.forward_pairs_q(CODEC, x, ids, tw, bank)
    out, ws = run_layer(x, ids, tw, bank)
    got = out.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref).any(axis=1)
    assert np.isfinite(got[fin]).all()
    err = rel_err_rows(got[fin], ref[fin])
    print(f"  max row rel err {err.max():.3e} over {fin.sum()} rows", flush=True)
    assert err.max() <= ARITH
    check_path(ws)


def test_mx8_sorted_prefill_full_size_sampled():
    # the prefill workload (E = 256, top-8, H = 4096, I = 2048) in mxfp8 at T = 512
    T = 512
    w = synth.WORKLOADS["prefill"]
    lay = synth.make_layer_q(CODEC, w, T, 0, seed=0, device="cuda")
    say("mxfp8 prefill", T, "u", lay.bank.E)
    out, ws = run_layer(lay.x, lay.ids, lay.weights, lay.bank)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    check_path(ws)
    sample = coverage_tokens(lay.ids, lay.bank.E, n=64, seed=T)
    used = np.unique(lay.ids[sample])
    sub = lay.bank.select(used).to("cpu")
    ref = oracle.forward_pairs_q(CODEC, lay.x[sample].cpu(), np.searchsorted(used, lay.ids[sample]).astype(np.int32),
                                 lay.weights[sample], sub)
    err = rel_err_rows(got[sample], ref)
    print(f"  sampled rows {sample}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= ARITH
