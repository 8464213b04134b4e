"""The forward call under HIP graph capture (needs an MI355X).

The library enqueues only kernel launches on the caller's stream (no
allocation, no synchronisation, no memset), so a captured forward must replay
to the eager result bit for bit.  Each replay is followed by eager work and a
synchronisation, and every replay is checked, on both paths.
"""

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _q():
    import quantized_expert_gather_amd as q
    return q


@pytest.mark.parametrize("shape", [(2, 8, 64, 1024, 256), (40, 4, 8, 256, 128)], ids=["union_L2", "sorted_T40"])
def test_forward_replays_under_graph_capture(shape):
    q = _q()
    L, k, E, H, I = shape
    x, ids, tw, bank = synth.random_problem(L, k, E, H, I, seed=21)
    print("[case] graph", shape, flush=True)
    dev = torch.device("cuda")
    xd, idd, twd, bk = x.to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev), bank.to(dev)
    ws = q.new_workspace(L, k, E, H, I, dev)
    out = torch.empty((L, H), dtype=torch.float32, device=dev)
    # eager reference (also warms the launch-configuration caches before capture)
    ref = q.forward_bank(xd, idd, twd, bk, out_dtype=torch.float32, workspace=ws).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            q.forward_bank(xd, idd, twd, bk, out=out, out_dtype=torch.float32, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        # eager work between replays: another forward into a separate buffer
        other = q.forward_bank(xd, idd, twd, bk, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
    assert np.isfinite(ref.cpu().numpy()).all()


def test_mxfp4_sorted_forward_replays_under_graph_capture():
    # the mxfp4 sorted path: folded pass, exact pass over the blocks it flags
    # (one expert's gate scales are subnormal, so the flags are set on every
    # replay), combine; replays checked against the eager result bit for bit
    q = _q()
    T, k, E, H, I = 48, 4, 6, 1024, 1024
    x, ids, tw, bank = synth.random_problem_mx(T, k, E, H, I, seed=22)
    bank.sg[2, :, ::3] = 0
    print("[case] graph mxfp4 sorted", (T, k, E, H, I), flush=True)
    dev = torch.device("cuda")
    xd, idd, twd, bk = x.to(dev), torch.from_numpy(ids).to(dev), torch.from_numpy(tw).to(dev), bank.to(dev)
    ws = torch.empty(q.moe_swiglu_mxfp4_workspace_bytes(T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ref = q.forward_bank_mx(xd, idd, twd, bk, out_dtype=torch.float32, workspace=ws).clone()
    torch.cuda.synchronize()
    assert q.moe_q4_read_device_status(ws) == (0, q.MOE_Q4_PATH_SORTED)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            q.forward_bank_mx(xd, idd, twd, bk, out=out, out_dtype=torch.float32, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        other = q.forward_bank_mx(xd, idd, twd, bk, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)
    assert np.isfinite(ref.cpu().numpy()).all()
