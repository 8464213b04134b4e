"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/moe_q4.h declares, and
reject invalid arguments on the host before any GPU work.  Pointers passed
here are fake, aligned addresses: every call below returns from the host-side
validation, which runs before any HIP call.
"""

import ctypes
import os
import re

import pytest

import quantized_expert_gather_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_q4.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def header_constants():
    vals = {}
    for name, val in re.findall(r"#define\s+(MOE_Q4_[A-Z_0-9]+)\s+([0-9]+)u?", open(HEADER).read()):
        vals[name] = int(val)
    return vals


def test_library_exports_every_declared_function():
    lib = q.lib()
    names = header_functions()
    assert len(names) >= 7
    assert sorted(names) == sorted(q.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_header():
    for name, val in header_constants().items():
        if hasattr(q, name):
            assert getattr(q, name) == val, name


# fake device pointers: distinct, 256-byte aligned, far apart
BASE = 1 << 40
STRIDE = 1 << 34


def fake(i):
    return BASE + i * STRIDE


def call(L=2, k=2, E=8, H=256, I=128, group=64, bits=4, out_dtype=0, ws_bytes=1 << 30, stages=3, ptrs=None,
         ws=None, out=None):
    p = [fake(i) for i in range(12)] if ptrs is None else ptrs
    return q.lib().moe_swiglu_q4_forward_stages(*p, L, k, E, H, I, group, bits,
                                               fake(13) if out is None else out, out_dtype,
                                               fake(14) if ws is None else ws, ws_bytes, stages, None)


def test_zero_tokens_is_ok_without_gpu():
    assert call(L=0) == q.MOE_Q4_OK
    assert q.moe_swiglu_q4_workspace_bytes(0, 2, 8, 256, 128) == 0
    assert q.moe_swiglu_q4_select_path(0, 2, 8, 256, 128) == q.MOE_Q4_PATH_NONE


@pytest.mark.parametrize("kw,status", [
    (dict(L=-1), q.MOE_Q4_ERR_SHAPE),
    (dict(k=0), q.MOE_Q4_ERR_SHAPE),
    (dict(E=0), q.MOE_Q4_ERR_SHAPE),
    (dict(k=9, E=8), q.MOE_Q4_ERR_SHAPE),
    (dict(H=0), q.MOE_Q4_ERR_SHAPE),
    (dict(H=250), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(I=96), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(group=32), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(bits=8), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(out_dtype=5), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(stages=0), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(stages=4), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(E=20000, k=2), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(ws_bytes=64), q.MOE_Q4_ERR_WORKSPACE),
])
def test_invalid_arguments_rejected_on_host(kw, status):
    assert call(**kw) == status


def test_null_pointers_rejected():
    for i in range(12):
        p = [fake(j) for j in range(12)]
        p[i] = 0
        assert call(ptrs=p) == q.MOE_Q4_ERR_NULL, i
    assert call(out=0) == q.MOE_Q4_ERR_NULL
    assert call(ws=0) == q.MOE_Q4_ERR_WORKSPACE


def test_misalignment_rejected():
    for i, a in [(0, 8), (3, 8), (6, 4), (9, 2), (1, 2), (4, 2)]:
        p = [fake(j) for j in range(12)]
        p[i] += a
        assert call(ptrs=p) == q.MOE_Q4_ERR_ALIGN, i
    assert call(ws=fake(14) + 128) == q.MOE_Q4_ERR_ALIGN
    assert call(out=fake(13) + 8) == q.MOE_Q4_ERR_ALIGN


def test_output_alias_rejected():
    assert call(out=fake(0)) == q.MOE_Q4_ERR_ALIAS          # out == x
    assert call(out=fake(14) + 256) == q.MOE_Q4_ERR_ALIAS   # inside the workspace
    assert call(out=fake(3) + 1024) == q.MOE_Q4_ERR_ALIAS   # inside wg


def test_path_selection_and_limits():
    assert q.moe_swiglu_q4_select_path(1, 8, 256, 6144, 2048) == q.MOE_Q4_PATH_UNION
    assert q.moe_swiglu_q4_select_path(8, 8, 256, 6144, 2048) == q.MOE_Q4_PATH_UNION
    assert q.moe_swiglu_q4_select_path(32, 8, 256, 2048, 512) == q.MOE_Q4_PATH_UNION
    assert q.moe_swiglu_q4_select_path(2, 2, 8, 256, 128) == q.MOE_Q4_PATH_UNION
    assert q.moe_swiglu_q4_select_path(3, 2, 8, 200, 128) == -q.MOE_Q4_ERR_UNSUPPORTED
    assert q.moe_swiglu_q4_select_path(2, 9, 8, 256, 128) == -q.MOE_Q4_ERR_SHAPE
    # past the 32-bit token masks (or the pair limit) the sorted path takes over
    assert q.moe_swiglu_q4_select_path(33, 8, 256, 2048, 512) == q.MOE_Q4_PATH_SORTED
    assert q.moe_swiglu_q4_select_path(512, 8, 256, 4096, 2048) == q.MOE_Q4_PATH_SORTED
    assert q.moe_swiglu_q4_select_path(2048, 8, 256, 4096, 2048) == q.MOE_Q4_PATH_SORTED
    assert q.moe_swiglu_q4_select_path(200, 2, 8, 256, 128) == q.MOE_Q4_PATH_SORTED
    assert q.moe_swiglu_q4_select_path(64, 8, 16385, 256, 128) == -q.MOE_Q4_ERR_UNSUPPORTED


def test_sorted_workspace_holds_its_scratch():
    for T, k, E, H, I in [(512, 8, 256, 4096, 2048), (2048, 8, 256, 4096, 2048), (100, 4, 16, 256, 128)]:
        P = T * k
        n = q.moe_swiglu_q4_workspace_bytes(T, k, E, H, I)
        assert n % 256 == 0
        # h as bf16 hi + lo, per-pair outputs in fp32, index arrays, per-token group sums
        assert n >= P * I * 4 + P * H * 4 + 3 * P * 4 + (E + 1) * 4 + T * (H // 64) * 4


def test_sort_tiles_max_bounds_every_schedule():
    import numpy as np
    import oracle
    rng = np.random.default_rng(5)
    for L, k, E, bm in [(7, 3, 5, 2), (64, 8, 16, 32), (33, 8, 256, 32), (512, 8, 256, 32), (40, 4, 8, 128)]:
        cap = q.moe_sort_pairs_tiles_max(L, k, E, bm)
        assert cap == L * k // bm + min(E, L * k) + 1
        for _ in range(20):
            ids = rng.integers(0, E, size=(L, k))
            if rng.random() < 0.3:
                ids[:] = rng.integers(0, E)  # everything on one expert
            tiles = oracle.expert_tiles(oracle.sorted_pairs(ids, E)["offsets"], bm)
            assert len(tiles) <= cap


def test_sort_pairs_host_validation():
    f = q.lib().moe_sort_pairs
    p = [fake(i) for i in range(7)]
    cap = q.moe_sort_pairs_tiles_max(64, 8, 256, 32)
    assert f(p[0], 0, 8, 256, 32, p[1], p[2], p[3], p[4], cap, p[5], p[6], None) == q.MOE_Q4_ERR_SHAPE
    assert f(p[0], 64, 8, 256, 0, p[1], p[2], p[3], p[4], cap, p[5], p[6], None) == q.MOE_Q4_ERR_SHAPE
    assert f(p[0], 64, 9, 8, 32, p[1], p[2], p[3], p[4], cap, p[5], p[6], None) == q.MOE_Q4_ERR_SHAPE
    assert f(0, 64, 8, 256, 32, p[1], p[2], p[3], p[4], cap, p[5], p[6], None) == q.MOE_Q4_ERR_NULL
    assert f(p[0], 64, 8, 256, 32, p[1], p[2], p[3], p[4], cap - 1, p[5], p[6], None) == q.MOE_Q4_ERR_WORKSPACE
    assert f(p[0], 64, 8, 256, 32, p[1], p[2], p[3], p[4] + 4, cap, p[5], p[6], None) == q.MOE_Q4_ERR_ALIGN
    assert f(p[0], 64, 8, 16385, 32, p[1], p[2], p[3], p[4], cap, p[5], p[6], None) == q.MOE_Q4_ERR_UNSUPPORTED


def test_workspace_size_grows_with_pairs():
    a = q.moe_swiglu_q4_workspace_bytes(1, 8, 256, 6144, 2048)
    b = q.moe_swiglu_q4_workspace_bytes(8, 8, 256, 6144, 2048)
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0
    # must hold the per-pair hidden (4 B per element) and output partials (4 B per element)
    assert b >= 64 * (2048 * 4 + 6144 * 4)


def test_route_union_host_validation():
    f = q.lib().moe_route_union
    ptr = [fake(i) for i in range(7)]
    assert f(ptr[0], ptr[1], 0, 8, 256, *ptr[2:], None) == q.MOE_Q4_ERR_SHAPE
    assert f(ptr[0], ptr[1], 33, 8, 256, *ptr[2:], None) == q.MOE_Q4_ERR_UNSUPPORTED
    assert f(ptr[0], ptr[1], 4, 9, 8, *ptr[2:], None) == q.MOE_Q4_ERR_SHAPE
    assert f(0, ptr[1], 4, 8, 256, *ptr[2:], None) == q.MOE_Q4_ERR_NULL
    assert f(ptr[0] + 2, ptr[1], 4, 8, 256, *ptr[2:], None) == q.MOE_Q4_ERR_ALIGN


def test_status_strings():
    for s in range(8):
        assert q.moe_q4_status_string(s)
    assert q.moe_q4_status_string(99) == "unknown status"


def test_binding_rejects_host_tensors_before_calling():
    import torch
    x = torch.zeros((2, 256), dtype=torch.bfloat16)
    ids = torch.zeros((2, 2), dtype=torch.int32)
    w = torch.zeros((2, 2), dtype=torch.float32)
    bank = [torch.zeros((8, 128, 32), dtype=torch.int32), torch.zeros((8, 128, 4), dtype=torch.bfloat16),
            torch.zeros((8, 128, 4), dtype=torch.bfloat16)] * 2 + \
           [torch.zeros((8, 256, 16), dtype=torch.int32), torch.zeros((8, 256, 2), dtype=torch.bfloat16),
            torch.zeros((8, 256, 2), dtype=torch.bfloat16)]
    with pytest.raises(ValueError):
        q.moe_swiglu_q4_forward(x, ids, w, *bank, workspace=torch.zeros(256, dtype=torch.uint8),
                                out=torch.zeros((2, 256), dtype=torch.bfloat16))


def call_mx(L=2, k=2, E=8, H=256, I=128, out_dtype=0, ws_bytes=1 << 30, stages=3, ptrs=None, ws=None, out=None):
    p = [fake(i) for i in range(9)] if ptrs is None else ptrs
    return q.lib().moe_swiglu_mxfp4_forward_stages(*p, L, k, E, H, I, fake(13) if out is None else out, out_dtype,
                                                  fake(14) if ws is None else ws, ws_bytes, stages, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=-1), q.MOE_Q4_ERR_SHAPE),
    (dict(k=9, E=8), q.MOE_Q4_ERR_SHAPE),
    (dict(H=0), q.MOE_Q4_ERR_SHAPE),
    (dict(H=240), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(I=112), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(L=33, stages=1), q.MOE_Q4_ERR_UNSUPPORTED),   # token chunks need all stages
    (dict(L=65536), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(k=1025, E=2048), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(out_dtype=5), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(stages=4), q.MOE_Q4_ERR_UNSUPPORTED),
    (dict(ws_bytes=64), q.MOE_Q4_ERR_WORKSPACE),
])
def test_mx_invalid_arguments_rejected_on_host(kw, status):
    assert call_mx(**kw) == status


def test_mx_host_checks():
    assert call_mx(L=0) == q.MOE_Q4_OK
    assert q.moe_swiglu_mxfp4_workspace_bytes(0, 2, 8, 256, 128) == 0
    # more tokens than one union launch, I not a multiple of 256 (so no sorted
    # path): the workspace of one 32-token chunk
    assert q.moe_swiglu_mxfp4_workspace_bytes(33, 8, 256, 2048, 480) == \
        q.moe_swiglu_mxfp4_workspace_bytes(32, 8, 256, 2048, 480) > 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(5000, 8, 256, 2048, 480) == \
        q.moe_swiglu_mxfp4_workspace_bytes(32, 8, 256, 2048, 480)
    assert q.moe_swiglu_mxfp4_workspace_bytes(100, 32, 256, 2048, 480) == \
        q.moe_swiglu_mxfp4_workspace_bytes(32, 32, 256, 2048, 480)
    # H and I multiples of 32 suffice; the layout is the union path's
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 96, 256) > 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 352, 224) > 0
    # the kernels' row steps: H <= 64 needs I % 64 == 0, I <= 128 needs H % 64 == 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 64, 32) == 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 96, 96) == 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 160, 128) == 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(2, 2, 4, 128, 128) > 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(8, 8, 256, 6144, 2048) == \
        q.moe_swiglu_q4_workspace_bytes(8, 8, 256, 6144, 2048)
    for i in range(9):
        p = [fake(j) for j in range(9)]
        p[i] = 0
        assert call_mx(ptrs=p) == q.MOE_Q4_ERR_NULL, i
    assert call_mx(ws=0) == q.MOE_Q4_ERR_WORKSPACE
    for i, a in [(0, 8), (3, 8), (5, 4), (7, 8), (1, 2), (2, 2)]:
        p = [fake(j) for j in range(9)]
        p[i] += a
        assert call_mx(ptrs=p) == q.MOE_Q4_ERR_ALIGN, i
    p = [fake(j) for j in range(9)]
    p[4] += 1  # scale bytes need no alignment
    assert call_mx(ptrs=p, ws=0) == q.MOE_Q4_ERR_WORKSPACE
    assert call_mx(out=fake(0)) == q.MOE_Q4_ERR_ALIAS
    assert call_mx(out=fake(8) + 64) == q.MOE_Q4_ERR_ALIAS   # inside sd
    assert call_mx(out=fake(14) + 256) == q.MOE_Q4_ERR_ALIAS


def test_mx_long_inputs_take_the_sorted_path_on_host():
    # more tokens than one union launch, H and I multiples of 256: the
    # sorted path's workspace (the layout the q4 sorted path uses)
    assert q.moe_swiglu_mxfp4_workspace_bytes(512, 8, 256, 4096, 2048) == \
        q.moe_swiglu_q4_workspace_bytes(512, 8, 256, 4096, 2048) > 0
    assert q.moe_swiglu_mxfp4_workspace_bytes(40, 8, 16, 4096, 1024) == \
        q.moe_swiglu_q4_workspace_bytes(40, 8, 16, 4096, 1024)
    assert q.moe_swiglu_mxfp4_workspace_bytes(512, 8, 256, 2048, 768) == \
        q.moe_swiglu_q4_workspace_bytes(512, 8, 256, 2048, 768)
    # widths that are not multiples of 256 stay on token chunks
    assert q.moe_swiglu_mxfp4_workspace_bytes(512, 8, 256, 2048, 480) == \
        q.moe_swiglu_mxfp4_workspace_bytes(32, 8, 256, 2048, 480)
    # the sorted path takes stage-only calls (host checks pass; with no GPU
    # the launch itself fails), token chunks do not
    n = q.moe_swiglu_mxfp4_workspace_bytes(40, 8, 16, 4096, 1024)
    assert call_mx(L=40, k=8, E=16, H=4096, I=1024, ws_bytes=n, stages=1) == q.MOE_Q4_ERR_LAUNCH
    assert call_mx(L=40, k=8, E=16, H=4096, I=480, stages=1) == q.MOE_Q4_ERR_UNSUPPORTED
    assert call_mx(L=40, k=8, E=16, H=4096, I=1024, ws_bytes=n - 1) == q.MOE_Q4_ERR_WORKSPACE
    # scale arrays the sorted path cannot read 8 bytes at a time: token chunks
    # where they fit, else an alignment error (H = 32768: not even one token
    # of a union launch fits the LDS)
    p = [fake(j) for j in range(9)]
    p[4] += 4
    assert call_mx(L=40, k=8, E=16, H=4096, I=1024, ws_bytes=n, ptrs=p, stages=1) == q.MOE_Q4_ERR_UNSUPPORTED
    assert call_mx(L=40, k=8, E=16, H=4096, I=1024, ws_bytes=n, ptrs=p) == q.MOE_Q4_ERR_LAUNCH
    assert q.moe_swiglu_codec_workspace_bytes(q.MOE_Q4_CODEC_NVFP4, 1, 8, 16, 32768, 1024) == 0
    m = q.moe_swiglu_mxfp4_workspace_bytes(40, 8, 16, 32768, 1024)
    assert m > 0
    assert call_mx(L=40, k=8, E=16, H=32768, I=1024, ws_bytes=m, ptrs=p) == q.MOE_Q4_ERR_ALIGN
    assert call_mx(L=40, k=8, E=16, H=32768, I=1024, ws_bytes=m) == q.MOE_Q4_ERR_LAUNCH


def test_mxfp8_long_inputs_take_the_sorted_path_on_host():
    m8 = q.MOE_Q4_CODEC_MXFP8
    assert q.moe_swiglu_codec_workspace_bytes(m8, 512, 8, 256, 4096, 2048) == \
        q.moe_swiglu_q4_workspace_bytes(512, 8, 256, 4096, 2048) > 0
    # not a multiple of 256: token chunks
    assert q.moe_swiglu_codec_workspace_bytes(m8, 512, 8, 256, 2048, 320) == \
        q.moe_swiglu_codec_workspace_bytes(m8, 32, 8, 256, 2048, 320)
    # the other codecs keep token chunks at multiples of 256 too
    for c in (q.MOE_Q4_CODEC_NVFP4, q.MOE_Q4_CODEC_AFFINE4_G32, q.MOE_Q4_CODEC_AFFINE8_G64):
        assert q.moe_swiglu_codec_workspace_bytes(c, 512, 8, 256, 2048, 1024) == \
            q.moe_swiglu_codec_workspace_bytes(c, 32, 8, 256, 2048, 1024), c


def test_codec_chunks_shrink_to_fit_the_lds():
    # H = 4096: 32 tokens' activations do not fit one workgroup's LDS, fewer do
    nv = q.MOE_Q4_CODEC_NVFP4
    assert q.moe_swiglu_codec_workspace_bytes(nv, 40, 8, 16, 4096, 256) > 0
    assert q.moe_swiglu_codec_workspace_bytes(nv, 40, 8, 16, 4096, 256) == \
        q.moe_swiglu_codec_workspace_bytes(nv, 5000, 8, 16, 4096, 256)
    assert q.moe_swiglu_codec_workspace_bytes(nv, 40, 8, 16, 4096, 256) < \
        q.moe_swiglu_codec_workspace_bytes(nv, 40, 8, 16, 2048, 256) * 2


def call_codec(codec, L=2, k=2, E=8, H=256, I=128, out_dtype=0, ws_bytes=1 << 30, stages=3, ptrs=None, ws=None,
               out=None):
    p = [fake(i) for i in range(12)] if ptrs is None else ptrs
    return q.lib().moe_swiglu_codec_forward_stages(codec, *p, L, k, E, H, I, fake(13) if out is None else out,
                                                  out_dtype, fake(14) if ws is None else ws, ws_bytes, stages, None)


def test_codec_host_checks():
    A32, MX, NV, A64 = q.MOE_Q4_CODEC_AFFINE4_G32, q.MOE_Q4_CODEC_MXFP4, q.MOE_Q4_CODEC_NVFP4, \
        q.MOE_Q4_CODEC_AFFINE4_G64
    assert call_codec(7) == q.MOE_Q4_ERR_UNSUPPORTED
    assert q.moe_swiglu_codec_workspace_bytes(7, 2, 2, 8, 256, 128) == 0
    for c in (A32, MX, NV):
        assert call_codec(c, L=0) == q.MOE_Q4_OK
        assert call_codec(c, H=240) == q.MOE_Q4_ERR_UNSUPPORTED
        assert call_codec(c, L=33, stages=2) == q.MOE_Q4_ERR_UNSUPPORTED
        assert call_codec(c, L=65536) == q.MOE_Q4_ERR_UNSUPPORTED
        assert call_codec(c, k=9) == q.MOE_Q4_ERR_SHAPE
        assert call_codec(c, ws_bytes=64) == q.MOE_Q4_ERR_WORKSPACE
        assert q.moe_swiglu_codec_workspace_bytes(c, 2, 2, 4, 96, 256) > 0
        assert q.moe_swiglu_codec_workspace_bytes(c, 8, 8, 256, 6144, 2048) == \
            q.moe_swiglu_q4_workspace_bytes(8, 8, 256, 6144, 2048)
    # codec 0 is moe_swiglu_q4_forward itself (H multiple of 64, sorted path above 32 tokens)
    assert q.moe_swiglu_codec_workspace_bytes(A64, 64, 8, 256, 4096, 2048) == \
        q.moe_swiglu_q4_workspace_bytes(64, 8, 256, 4096, 2048) > 0
    assert call_codec(A64, H=96) == q.MOE_Q4_ERR_UNSUPPORTED
    # biases: required for affine group 32, ignored by the FP4 codecs
    for i in (5, 8, 11):
        p = [fake(j) for j in range(12)]
        p[i] = 0
        assert call_codec(A32, ptrs=p) == q.MOE_Q4_ERR_NULL, i
        assert call_codec(NV, ptrs=p, ws=0) == q.MOE_Q4_ERR_WORKSPACE, i
    # scale alignment: 2 bytes for affine group 32 and nvfp4, none for mxfp4
    for c, want in ((A32, q.MOE_Q4_ERR_ALIGN), (NV, q.MOE_Q4_ERR_ALIGN), (MX, q.MOE_Q4_ERR_WORKSPACE)):
        p = [fake(j) for j in range(12)]
        p[7] += 1
        assert call_codec(c, ptrs=p, ws=0 if want != q.MOE_Q4_ERR_ALIGN else None) == want, c
    # out inside a bias array aliases for affine group 32 only
    assert call_codec(A32, out=fake(5) + 64) == q.MOE_Q4_ERR_ALIAS
    assert call_codec(NV, out=fake(5) + 64, ws=0) == q.MOE_Q4_ERR_WORKSPACE
    assert call_codec(NV, out=fake(10) + 64) == q.MOE_Q4_ERR_ALIAS


def test_codec_8bit_host_checks():
    A8, MX8 = q.MOE_Q4_CODEC_AFFINE8_G64, q.MOE_Q4_CODEC_MXFP8
    # group 64 for the 8-bit affine codes, 32 for mxfp8
    assert call_codec(A8, H=288) == q.MOE_Q4_ERR_UNSUPPORTED
    assert call_codec(A8, I=96) == q.MOE_Q4_ERR_UNSUPPORTED
    assert q.moe_swiglu_codec_workspace_bytes(A8, 2, 2, 4, 320, 128) > 0
    assert q.moe_swiglu_codec_workspace_bytes(MX8, 2, 2, 4, 96, 256) > 0
    assert q.moe_swiglu_codec_workspace_bytes(A8, 8, 8, 256, 6144, 2048) == \
        q.moe_swiglu_q4_workspace_bytes(8, 8, 256, 6144, 2048)
    # biases required for the 8-bit affine codes only; E8M0 scales need no alignment
    p = [fake(j) for j in range(12)]
    p[5] = 0
    assert call_codec(A8, ptrs=p) == q.MOE_Q4_ERR_NULL
    assert call_codec(MX8, ptrs=p, ws=0) == q.MOE_Q4_ERR_WORKSPACE
    p = [fake(j) for j in range(12)]
    p[4] += 1
    assert call_codec(A8, ptrs=p) == q.MOE_Q4_ERR_ALIGN
    assert call_codec(MX8, ptrs=p, ws=0) == q.MOE_Q4_ERR_WORKSPACE
    # 8-bit codes are twice the bytes: out just past the 4-bit size of wg still aliases
    assert call_codec(A8, out=fake(3) + 8 * 128 * 256 // 2 + 64) == q.MOE_Q4_ERR_ALIAS


def test_kernel_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    # the stored traffic figures stay valid across comment edits, not code edits
    import bench
    d = tmp_path / "quantized_expert_gather_amd" / "csrc"
    d.mkdir(parents=True)
    src = d / "k.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src.write_text("int f(int a) { return a + 1; }  // one\n")
    h0 = bench.kernel_source_hash()
    src.write_text("/* block\\n comment */\nint f(int a) {\n  return a + 1;  // changed comment\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asking for more exits at once with a message (no GPU touched)
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
