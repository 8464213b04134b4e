"""The allocation-free entry point against the ordinary one (needs an MI355X).

moe_swiglu_q4_forward_noalloc runs the same kernels as moe_swiglu_q4_forward
with the library's static scratch as the workspace, so its outputs must equal
the ordinary entry point's bit for bit.  Two calls in a row, the second with a
smaller input, check that the scratch left by one call does not leak into the
next; an input larger than the scratch is refused on the host.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _q():
    import quantized_expert_gather_amd as q
    return q


def _run_both(L, k, E, H, I, seed, out_dtype):
    q = _q()
    x, ids, tw, bank = synth.random_problem(L, k, E, H, I, seed=seed)
    dev = torch.device("cuda")
    xd, idd, twd, bk = x.to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev), bank.to(dev)
    ref = q.forward_bank(xd, idd, twd, bk, out_dtype=out_dtype)
    out = torch.full((L, H), float("nan"), dtype=out_dtype, device=dev)
    q.moe_swiglu_q4_forward_noalloc(xd, idd, twd, *bk.tensors(), out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_matches_forward_twice_shrinking(out_dtype):
    # first call: 8 tokens (union path, combine kernel); second: 3 tokens on a
    # smaller bank; third: one token (the down kernel writes out itself)
    for (L, k, E, H, I, seed) in ((8, 8, 48, 2048, 512, 41), (3, 4, 12, 1024, 256, 42), (1, 8, 16, 2048, 512, 43)):
        print("[case] noalloc L=%d k=%d E=%d H=%d I=%d" % (L, k, E, H, I), out_dtype, flush=True)
        ref, out = _run_both(L, k, E, H, I, seed, out_dtype)
        assert torch.equal(ref.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))


def test_noalloc_verify_layer_then_smaller():
    # a full-size GLM-5.2-style verify layer at L = 8, then at L = 2
    q = _q()
    w = synth.WORKLOADS["verify"]
    for L, layer in ((8, 12), (2, 50)):
        print("[case] noalloc verify L=%d layer %d" % (L, layer), flush=True)
        lay = synth.make_layer(w, L, layer, seed=0, device="cuda")
        idd = torch.from_numpy(lay.ids).cuda()
        twd = torch.from_numpy(lay.weights).cuda()
        ref = q.forward_bank(lay.x, idd, twd, lay.bank, out_dtype=torch.float32)
        out = torch.empty((L, w.H), dtype=torch.float32, device="cuda")
        q.moe_swiglu_q4_forward_noalloc(lay.x, idd, twd, *lay.bank.tensors(), out)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), out.view(torch.int32))


def test_noalloc_refuses_inputs_beyond_the_scratch():
    q = _q()
    L, k, E, H, I = 512, 8, 16, 1024, 256  # sorted path, workspace well above 16 MiB
    assert q.moe_swiglu_q4_workspace_bytes(L, k, E, H, I) > q.MOE_Q4_NOALLOC_SCRATCH_BYTES
    x, ids, tw, bank = synth.random_problem(L, k, E, H, I, seed=44)
    dev = torch.device("cuda")
    out = torch.zeros((L, H), dtype=torch.float32, device=dev)
    with pytest.raises(q.MoeQ4Error) as ei:
        q.moe_swiglu_q4_forward_noalloc(x.to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev),
                                        *bank.to(dev).tensors(), out)
    assert ei.value.status == q.MOE_Q4_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (out == 0).all()
