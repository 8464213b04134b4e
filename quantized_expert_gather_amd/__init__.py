"""Python binding of libmoe_q4.so, the MI355X SwitchGLU-q4 MoE library.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/moe_q4.h``.  PyTorch supplies device
memory and the current stream.  If the built library is missing this module
raises on first use; there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_q4.so")

MOE_Q4_OK = 0
MOE_Q4_ERR_NULL = 1
MOE_Q4_ERR_SHAPE = 2
MOE_Q4_ERR_UNSUPPORTED = 3
MOE_Q4_ERR_ALIGN = 4
MOE_Q4_ERR_WORKSPACE = 5
MOE_Q4_ERR_LAUNCH = 6
MOE_Q4_ERR_ALIAS = 7
MOE_Q4_ERR_SCRATCH = 8
MOE_Q4_DEV_BAD_ID = 1
MOE_Q4_OUT_BF16 = 0
MOE_Q4_OUT_F32 = 1
MOE_Q4_PATH_NONE = 0
MOE_Q4_PATH_UNION = 1
MOE_Q4_PATH_SORTED = 2
MOE_Q4_STAGE_GATEUP = 1
MOE_Q4_STAGE_DOWN = 2
MOE_Q4_STAGE_ALL = 3
MOE_Q4_CODEC_AFFINE4_G64 = 0
MOE_Q4_CODEC_AFFINE4_G32 = 1
MOE_Q4_CODEC_MXFP4 = 2
MOE_Q4_CODEC_NVFP4 = 3
MOE_Q4_CODEC_AFFINE8_G64 = 4
MOE_Q4_CODEC_MXFP8 = 5
#: codec names (as in the test-data generators) -> MOE_Q4_CODEC_*, inputs per scale group, bits per code
CODECS = {"affine4_g64": (MOE_Q4_CODEC_AFFINE4_G64, 64, 4), "affine4_g32": (MOE_Q4_CODEC_AFFINE4_G32, 32, 4),
          "mxfp4": (MOE_Q4_CODEC_MXFP4, 32, 4), "nvfp4": (MOE_Q4_CODEC_NVFP4, 16, 4),
          "affine8_g64": (MOE_Q4_CODEC_AFFINE8_G64, 64, 8), "mxfp8": (MOE_Q4_CODEC_MXFP8, 32, 8)}
MOE_Q4_UNION_MAX_L = 32
MOE_Q4_MAX_PAIRS = 1024
MOE_Q4_CODEC_MAX_L = 65535
MOE_Q4_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTS = (
    "moe_swiglu_q4_workspace_bytes",
    "moe_swiglu_q4_select_path",
    "moe_swiglu_q4_forward",
    "moe_swiglu_q4_forward_stages",
    "moe_swiglu_q4_forward_noalloc",
    "moe_swiglu_codec_workspace_bytes",
    "moe_swiglu_codec_forward",
    "moe_swiglu_codec_forward_stages",
    "moe_swiglu_mxfp4_workspace_bytes",
    "moe_swiglu_mxfp4_forward",
    "moe_swiglu_mxfp4_forward_stages",
    "moe_route_union",
    "moe_sort_pairs_tiles_max",
    "moe_sort_pairs",
    "moe_q4_read_device_status",
    "moe_q4_clear_device_status",
    "moe_q4_status_string",
    "moe_q4_stream_read",
)

_lib = None


class MoeQ4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({moe_q4_status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_expert_gather_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, U = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint
    L.moe_swiglu_q4_workspace_bytes.argtypes = [I32] * 5
    L.moe_swiglu_q4_workspace_bytes.restype = SZ
    L.moe_swiglu_q4_select_path.argtypes = [I32] * 5
    L.moe_swiglu_q4_select_path.restype = I32
    fwd = [P] * 12 + [I32] * 7 + [P, I32, P, SZ]
    L.moe_swiglu_q4_forward.argtypes = fwd + [P]
    L.moe_swiglu_q4_forward.restype = I32
    L.moe_swiglu_q4_forward_stages.argtypes = fwd + [U, P]
    L.moe_swiglu_q4_forward_stages.restype = I32
    L.moe_swiglu_q4_forward_noalloc.argtypes = [P] * 12 + [I32] * 7 + [P, I32, P]
    L.moe_swiglu_q4_forward_noalloc.restype = I32
    L.moe_swiglu_codec_workspace_bytes.argtypes = [I32] * 6
    L.moe_swiglu_codec_workspace_bytes.restype = SZ
    fwd_c = [I32] + [P] * 12 + [I32] * 5 + [P, I32, P, SZ]
    L.moe_swiglu_codec_forward.argtypes = fwd_c + [P]
    L.moe_swiglu_codec_forward.restype = I32
    L.moe_swiglu_codec_forward_stages.argtypes = fwd_c + [U, P]
    L.moe_swiglu_codec_forward_stages.restype = I32
    L.moe_swiglu_mxfp4_workspace_bytes.argtypes = [I32] * 5
    L.moe_swiglu_mxfp4_workspace_bytes.restype = SZ
    fwd_mx = [P] * 9 + [I32] * 5 + [P, I32, P, SZ]
    L.moe_swiglu_mxfp4_forward.argtypes = fwd_mx + [P]
    L.moe_swiglu_mxfp4_forward.restype = I32
    L.moe_swiglu_mxfp4_forward_stages.argtypes = fwd_mx + [U, P]
    L.moe_swiglu_mxfp4_forward_stages.restype = I32
    L.moe_route_union.argtypes = [P, P, I32, I32, I32, P, P, P, P, P, P]
    L.moe_route_union.restype = I32
    L.moe_sort_pairs_tiles_max.argtypes = [I32] * 4
    L.moe_sort_pairs_tiles_max.restype = I32
    L.moe_sort_pairs.argtypes = [P, I32, I32, I32, I32, P, P, P, P, I32, P, P, P]
    L.moe_sort_pairs.restype = I32
    L.moe_q4_read_device_status.argtypes = [P, P, P, P]
    L.moe_q4_read_device_status.restype = I32
    L.moe_q4_clear_device_status.argtypes = [P, P]
    L.moe_q4_clear_device_status.restype = I32
    L.moe_q4_status_string.argtypes = [I32]
    L.moe_q4_status_string.restype = ctypes.c_char_p
    L.moe_q4_stream_read.argtypes = [P, SZ, P, SZ, P]
    L.moe_q4_stream_read.restype = I32
    _lib = L
    return L


def moe_q4_status_string(status: int) -> str:
    try:
        return lib().moe_q4_status_string(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def _stream_ptr(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev_ptr(t: Optional[torch.Tensor], dtypes, name: str) -> int:
    if t is None:
        return 0
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _check(status: int, where: str) -> None:
    if status != MOE_Q4_OK:
        raise MoeQ4Error(status, where)


def moe_swiglu_q4_workspace_bytes(L: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_swiglu_q4_workspace_bytes(L, k, E, H, I))


def moe_swiglu_q4_select_path(L: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_swiglu_q4_select_path(L, k, E, H, I))


def new_workspace(L: int, k: int, E: int, H: int, I: int, device=None) -> torch.Tensor:
    """A workspace for this shape (its contents need no initialisation)."""
    n = moe_swiglu_q4_workspace_bytes(L, k, E, H, I)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


_I32 = (torch.int32,)
_U32 = (torch.int32, getattr(torch, "uint32", torch.int32))
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)


def moe_swiglu_q4_forward(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, out=None,
                          out_dtype=torch.bfloat16, workspace=None, stream=None,
                          stages: int = MOE_Q4_STAGE_ALL) -> torch.Tensor:
    """One SwitchGLU-q4 MoE layer (see include/moe_q4.h for the contract).

    x bf16 [L, H]; topk_ids int32 [L, k]; topk_weights fp32 [L, k];
    wg/wu int32 (uint32 bits) [E, I, H/8]; sg/bg/su/bu bf16 [E, I, H/64];
    wd int32 [E, H, I/8]; sd/bd bf16 [E, H, I/64].  Returns out [L, H].
    """
    if x.dim() != 2 or topk_ids.dim() != 2 or wg.dim() != 3 or wd.dim() != 3:
        raise ValueError("x [L, H], topk_ids [L, k], wg [E, I, H/8] and wd [E, H, I/8] expected")
    L, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg.shape[0], wg.shape[1]
    shapes = {
        "topk_ids": (topk_ids, (L, k)), "topk_weights": (topk_weights, (L, k)),
        "wg": (wg, (E, I, H // 8)), "wu": (wu, (E, I, H // 8)), "wd": (wd, (E, H, I // 8)),
        "sg": (sg, (E, I, H // 64)), "bg": (bg, (E, I, H // 64)), "su": (su, (E, I, H // 64)),
        "bu": (bu, (E, I, H // 64)), "sd": (sd, (E, H, I // 64)), "bd": (bd, (E, H, I // 64)),
    }
    for name, (t, shp) in shapes.items():
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    od = MOE_Q4_OUT_F32 if out_dtype == torch.float32 else MOE_Q4_OUT_BF16
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32 if od == MOE_Q4_OUT_F32 else torch.bfloat16, device=x.device)
    if tuple(out.shape) != (L, H):
        raise ValueError("out must be [L, H]")
    if workspace is None:
        workspace = new_workspace(L, k, E, H, I, x.device)
    st = lib().moe_swiglu_q4_forward_stages(
        _dev_ptr(x, _BF16, "x"), _dev_ptr(topk_ids, _I32, "topk_ids"), _dev_ptr(topk_weights, _F32, "topk_weights"),
        _dev_ptr(wg, _U32, "wg"), _dev_ptr(sg, _BF16, "sg"), _dev_ptr(bg, _BF16, "bg"),
        _dev_ptr(wu, _U32, "wu"), _dev_ptr(su, _BF16, "su"), _dev_ptr(bu, _BF16, "bu"),
        _dev_ptr(wd, _U32, "wd"), _dev_ptr(sd, _BF16, "sd"), _dev_ptr(bd, _BF16, "bd"),
        L, k, E, H, I, 64, 4,
        _dev_ptr(out, (torch.float32,) if od == MOE_Q4_OUT_F32 else _BF16, "out"), od,
        _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(),
        int(stages), _stream_ptr(stream))
    _check(st, "moe_swiglu_q4_forward")
    return out


def moe_swiglu_q4_forward_noalloc(x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, out,
                                  stream=None) -> torch.Tensor:
    """The layer through the allocation-free entry point: no workspace
    argument (the library's static scratch serves as one) and a caller-owned
    ``out`` (bf16 or fp32 [L, H]); shapes as for :func:`moe_swiglu_q4_forward`."""
    L, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg.shape[0], wg.shape[1]
    od = MOE_Q4_OUT_F32 if out.dtype == torch.float32 else MOE_Q4_OUT_BF16
    if tuple(out.shape) != (L, H):
        raise ValueError("out must be [L, H]")
    st = lib().moe_swiglu_q4_forward_noalloc(
        _dev_ptr(x, _BF16, "x"), _dev_ptr(topk_ids, _I32, "topk_ids"), _dev_ptr(topk_weights, _F32, "topk_weights"),
        _dev_ptr(wg, _U32, "wg"), _dev_ptr(sg, _BF16, "sg"), _dev_ptr(bg, _BF16, "bg"),
        _dev_ptr(wu, _U32, "wu"), _dev_ptr(su, _BF16, "su"), _dev_ptr(bu, _BF16, "bu"),
        _dev_ptr(wd, _U32, "wd"), _dev_ptr(sd, _BF16, "sd"), _dev_ptr(bd, _BF16, "bd"),
        L, k, E, H, I, 64, 4,
        _dev_ptr(out, (torch.float32,) if od == MOE_Q4_OUT_F32 else _BF16, "out"), od, _stream_ptr(stream))
    _check(st, "moe_swiglu_q4_forward_noalloc")
    return out


def forward_bank(x, topk_ids, topk_weights, bank, **kw) -> torch.Tensor:
    """moe_swiglu_q4_forward with the nine bank tensors taken from an object
    exposing ``tensors()`` (wg, sg, bg, wu, su, bu, wd, sd, bd)."""
    return moe_swiglu_q4_forward(x, topk_ids, topk_weights, *bank.tensors(), **kw)


def moe_swiglu_mxfp4_workspace_bytes(L: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_swiglu_mxfp4_workspace_bytes(L, k, E, H, I))


_U8 = (torch.uint8,)


def moe_swiglu_mxfp4_forward(x, topk_ids, topk_weights, wg, sg, wu, su, wd, sd, out=None,
                             out_dtype=torch.bfloat16, workspace=None, stream=None,
                             stages: int = MOE_Q4_STAGE_ALL) -> torch.Tensor:
    """One SwitchGLU MoE layer over mxfp4 banks (see include/moe_q4.h).

    x bf16 [L, H]; topk_ids int32 [L, k]; topk_weights fp32 [L, k];
    wg/wu int32 (uint32 bits) [E, I, H/8]; sg/su uint8 E8M0 [E, I, H/32];
    wd int32 [E, H, I/8]; sd uint8 [E, H, I/32].  Returns out [L, H].
    """
    if x.dim() != 2 or topk_ids.dim() != 2 or wg.dim() != 3 or wd.dim() != 3:
        raise ValueError("x [L, H], topk_ids [L, k], wg [E, I, H/8] and wd [E, H, I/8] expected")
    L, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg.shape[0], wg.shape[1]
    shapes = {
        "topk_ids": (topk_ids, (L, k)), "topk_weights": (topk_weights, (L, k)),
        "wg": (wg, (E, I, H // 8)), "wu": (wu, (E, I, H // 8)), "wd": (wd, (E, H, I // 8)),
        "sg": (sg, (E, I, H // 32)), "su": (su, (E, I, H // 32)), "sd": (sd, (E, H, I // 32)),
    }
    for name, (t, shp) in shapes.items():
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    od = MOE_Q4_OUT_F32 if out_dtype == torch.float32 else MOE_Q4_OUT_BF16
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32 if od == MOE_Q4_OUT_F32 else torch.bfloat16, device=x.device)
    if tuple(out.shape) != (L, H):
        raise ValueError("out must be [L, H]")
    if workspace is None:
        n = moe_swiglu_mxfp4_workspace_bytes(L, k, E, H, I)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    st = lib().moe_swiglu_mxfp4_forward_stages(
        _dev_ptr(x, _BF16, "x"), _dev_ptr(topk_ids, _I32, "topk_ids"), _dev_ptr(topk_weights, _F32, "topk_weights"),
        _dev_ptr(wg, _U32, "wg"), _dev_ptr(sg, _U8, "sg"), _dev_ptr(wu, _U32, "wu"), _dev_ptr(su, _U8, "su"),
        _dev_ptr(wd, _U32, "wd"), _dev_ptr(sd, _U8, "sd"), L, k, E, H, I,
        _dev_ptr(out, (torch.float32,) if od == MOE_Q4_OUT_F32 else _BF16, "out"), od,
        _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(),
        int(stages), _stream_ptr(stream))
    _check(st, "moe_swiglu_mxfp4_forward")
    return out


def moe_swiglu_codec_workspace_bytes(codec: int, L: int, k: int, E: int, H: int, I: int) -> int:
    return int(lib().moe_swiglu_codec_workspace_bytes(int(codec), L, k, E, H, I))


def _codec_id(codec) -> int:
    return CODECS[codec][0] if isinstance(codec, str) else int(codec)


def _codec_args(codec_name, x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd):
    """Shape- and dtype-checked pointer list of a codec call."""
    code = _codec_id(codec_name)
    spec = {v[0]: v[1:] for v in CODECS.values()}.get(code)
    if spec is None:
        raise ValueError(f"unknown codec {codec_name!r}")
    gs, bits = spec
    if x.dim() != 2 or topk_ids.dim() != 2 or wg.dim() != 3 or wd.dim() != 3:
        raise ValueError("x [L, H], topk_ids [L, k], wg [E, I, H/8] and wd [E, H, I/8] expected")
    L, H = x.shape
    k = topk_ids.shape[1]
    E, I = wg.shape[0], wg.shape[1]
    affine = code in (MOE_Q4_CODEC_AFFINE4_G64, MOE_Q4_CODEC_AFFINE4_G32, MOE_Q4_CODEC_AFFINE8_G64)
    per_word = 32 // bits
    if wg.shape[2] * per_word != H:
        raise ValueError(f"wg has {wg.shape[2]} words per row, expected {H // per_word}")
    shapes = {
        "topk_ids": (topk_ids, (L, k)), "topk_weights": (topk_weights, (L, k)),
        "wg": (wg, (E, I, H // per_word)), "wu": (wu, (E, I, H // per_word)), "wd": (wd, (E, H, I // per_word)),
        "sg": (sg, (E, I, H // gs)), "su": (su, (E, I, H // gs)), "sd": (sd, (E, H, I // gs)),
    }
    if affine:
        shapes.update({"bg": (bg, (E, I, H // gs)), "bu": (bu, (E, I, H // gs)), "bd": (bd, (E, H, I // gs))})
    for name, (t, shp) in shapes.items():
        if t is None or tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {None if t is None else tuple(t.shape)}, expected {shp}")
    st = _BF16 if affine else _U8
    ptrs = [_dev_ptr(x, _BF16, "x"), _dev_ptr(topk_ids, _I32, "topk_ids"),
            _dev_ptr(topk_weights, _F32, "topk_weights"),
            _dev_ptr(wg, _U32, "wg"), _dev_ptr(sg, st, "sg"), _dev_ptr(bg, _BF16, "bg") if affine else 0,
            _dev_ptr(wu, _U32, "wu"), _dev_ptr(su, st, "su"), _dev_ptr(bu, _BF16, "bu") if affine else 0,
            _dev_ptr(wd, _U32, "wd"), _dev_ptr(sd, st, "sd"), _dev_ptr(bd, _BF16, "bd") if affine else 0]
    return code, ptrs, (L, k, E, H, I)


def moe_swiglu_codec_forward(codec, x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd, out=None,
                             out_dtype=torch.bfloat16, workspace=None, stream=None,
                             stages: int = MOE_Q4_STAGE_ALL) -> torch.Tensor:
    """One SwitchGLU MoE layer over a bank in ``codec`` (a name of :data:`CODECS`
    or a MOE_Q4_CODEC_* value; see include/moe_q4.h).  Scales are bf16 for
    the affine codecs and uint8 otherwise; biases are bf16 for the affine
    codecs and ignored (may be None) otherwise."""
    code, ptrs, (L, k, E, H, I) = _codec_args(codec, x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd)
    od = MOE_Q4_OUT_F32 if out_dtype == torch.float32 else MOE_Q4_OUT_BF16
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32 if od == MOE_Q4_OUT_F32 else torch.bfloat16, device=x.device)
    if tuple(out.shape) != (L, H):
        raise ValueError("out must be [L, H]")
    if workspace is None:
        n = moe_swiglu_codec_workspace_bytes(code, L, k, E, H, I)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
    st = lib().moe_swiglu_codec_forward_stages(
        code, *ptrs, L, k, E, H, I, _dev_ptr(out, (torch.float32,) if od == MOE_Q4_OUT_F32 else _BF16, "out"), od,
        _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), int(stages), _stream_ptr(stream))
    _check(st, "moe_swiglu_codec_forward")
    return out


def forward_bank_codec(x, topk_ids, topk_weights, bank, **kw) -> torch.Tensor:
    """moe_swiglu_codec_forward with the codec and the nine bank tensors taken
    from an object exposing ``codec`` and ``tensors()`` (wg, sg, bg, wu, su,
    bu, wd, sd, bd; biases None for the codecs without one)."""
    return moe_swiglu_codec_forward(bank.codec, x, topk_ids, topk_weights, *bank.tensors(), **kw)


def forward_bank_mx(x, topk_ids, topk_weights, bank, **kw) -> torch.Tensor:
    """moe_swiglu_mxfp4_forward with the six bank tensors taken from an object
    exposing ``tensors()`` (wg, sg, wu, su, wd, sd)."""
    return moe_swiglu_mxfp4_forward(x, topk_ids, topk_weights, *bank.tensors(), **kw)


def moe_route_union(topk_ids: torch.Tensor, topk_weights: torch.Tensor, E: int, stream=None) -> Dict[str, torch.Tensor]:
    """Distinct experts of the routes (see include/moe_q4.h).  Returns device tensors."""
    L, k = topk_ids.shape
    u_max = min(E, L * k)
    dev = topk_ids.device
    res = {
        "u": torch.empty(1, dtype=torch.int32, device=dev),
        "uniq_ids": torch.empty(max(u_max, 1), dtype=torch.int32, device=dev),
        "tok_mask": torch.empty(max(u_max, 1), dtype=torch.int32, device=dev),
        "uniq_w": torch.empty((max(u_max, 1), L), dtype=torch.float32, device=dev),
        "slot_to_uniq": torch.empty((L, k), dtype=torch.int32, device=dev),
    }
    st = lib().moe_route_union(_dev_ptr(topk_ids, _I32, "topk_ids"), _dev_ptr(topk_weights, _F32, "topk_weights"),
                               L, k, E, res["u"].data_ptr(), res["uniq_ids"].data_ptr(), res["tok_mask"].data_ptr(),
                               res["uniq_w"].data_ptr(), res["slot_to_uniq"].data_ptr(), _stream_ptr(stream))
    _check(st, "moe_route_union")
    return res


def moe_sort_pairs_tiles_max(L: int, k: int, E: int, bm: int) -> int:
    n = int(lib().moe_sort_pairs_tiles_max(L, k, E, bm))
    if n < 0:
        raise MoeQ4Error(-n, "moe_sort_pairs_tiles_max")
    return n


def moe_sort_pairs(topk_ids: torch.Tensor, E: int, bm: int, stream=None) -> Dict[str, torch.Tensor]:
    """Expert sort of the pairs and the row-tile list (see include/moe_q4.h).  Returns device tensors;
    ``tiles`` holds all ``tiles_max`` rows, of which ``info[3]`` are written."""
    L, k = topk_ids.shape
    P = L * k
    cap = moe_sort_pairs_tiles_max(L, k, E, bm)
    dev = topk_ids.device
    res = {
        "offsets": torch.empty(E + 1, dtype=torch.int32, device=dev),
        "perm": torch.empty(max(P, 1), dtype=torch.int32, device=dev),
        "inv": torch.empty(max(P, 1), dtype=torch.int32, device=dev),
        "tiles": torch.empty((cap, 4), dtype=torch.int32, device=dev),
        "info": torch.empty(4, dtype=torch.int32, device=dev),
    }
    scratch = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    st = lib().moe_sort_pairs(_dev_ptr(topk_ids, _I32, "topk_ids"), L, k, E, bm, res["offsets"].data_ptr(),
                              res["perm"].data_ptr(), res["inv"].data_ptr(), res["tiles"].data_ptr(), cap,
                              res["info"].data_ptr(), scratch.data_ptr(), _stream_ptr(stream))
    _check(st, "moe_sort_pairs")
    res["_scratch"] = scratch  # kept alive until the caller has synchronised
    return res


def moe_q4_read_device_status(workspace: torch.Tensor, stream=None) -> Tuple[int, int]:
    """(status bits, path) of the last forward that used this workspace; synchronises the stream."""
    st_v = ctypes.c_uint32(0)
    path_v = ctypes.c_uint32(0)
    st = lib().moe_q4_read_device_status(_dev_ptr(workspace, (torch.uint8,), "workspace"), ctypes.byref(st_v),
                                         ctypes.byref(path_v), _stream_ptr(stream))
    _check(st, "moe_q4_read_device_status")
    return int(st_v.value), int(path_v.value)


def moe_q4_clear_device_status(workspace: torch.Tensor, stream=None) -> None:
    _check(lib().moe_q4_clear_device_status(_dev_ptr(workspace, (torch.uint8,), "workspace"), _stream_ptr(stream)),
           "moe_q4_clear_device_status")


class PreparedForward:
    """A forward (or stage) call whose arguments were checked and marshalled
    once; calling it only crosses the C ABI.  The tensors must stay alive and
    unchanged in place for as long as the object is used."""

    def __init__(self, x, topk_ids, topk_weights, bank_tensors, out, workspace, stages=MOE_Q4_STAGE_ALL,
                 stream=None):
        wg, sg, bg, wu, su, bu, wd, sd, bd = bank_tensors
        # one checked call through the normal path validates shapes and dtypes
        self._keep = (x, topk_ids, topk_weights, tuple(bank_tensors), out, workspace)
        L, H = x.shape
        k = topk_ids.shape[1]
        E, I = wg.shape[0], wg.shape[1]
        od = MOE_Q4_OUT_F32 if out.dtype == torch.float32 else MOE_Q4_OUT_BF16
        ptrs = [_dev_ptr(t, _BF16 if i in (0,) else (_I32 if i == 1 else (_F32 if i == 2 else
                                                                            (_U32 if i in (3, 6, 9) else _BF16))),
                         "arg%d" % i)
                for i, t in enumerate((x, topk_ids, topk_weights, wg, sg, bg, wu, su, bu, wd, sd, bd))]
        self._args = (*ptrs, L, k, E, H, I, 64, 4, _dev_ptr(out, (out.dtype,), "out"), od,
                      _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), int(stages),
                      _stream_ptr(stream))
        self._fn = lib().moe_swiglu_q4_forward_stages

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st:
            raise MoeQ4Error(st, "moe_swiglu_q4_forward_stages")


class PreparedForwardMX:
    """:class:`PreparedForward` for mxfp4 banks (wg, sg, wu, su, wd, sd)."""

    def __init__(self, x, topk_ids, topk_weights, bank_tensors, out, workspace, stages=MOE_Q4_STAGE_ALL,
                 stream=None):
        wg, sg, wu, su, wd, sd = bank_tensors
        self._keep = (x, topk_ids, topk_weights, tuple(bank_tensors), out, workspace)
        L, H = x.shape
        k = topk_ids.shape[1]
        E, I = wg.shape[0], wg.shape[1]
        od = MOE_Q4_OUT_F32 if out.dtype == torch.float32 else MOE_Q4_OUT_BF16
        kinds = (_BF16, _I32, _F32, _U32, _U8, _U32, _U8, _U32, _U8)
        ptrs = [_dev_ptr(t, kd, "arg%d" % i)
                for i, (t, kd) in enumerate(zip((x, topk_ids, topk_weights, wg, sg, wu, su, wd, sd), kinds))]
        self._args = (*ptrs, L, k, E, H, I, _dev_ptr(out, (out.dtype,), "out"), od,
                      _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), int(stages),
                      _stream_ptr(stream))
        self._fn = lib().moe_swiglu_mxfp4_forward_stages

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st:
            raise MoeQ4Error(st, "moe_swiglu_mxfp4_forward_stages")


class PreparedForwardCodec:
    """:class:`PreparedForward` for any codec (bank tensors as for
    :func:`moe_swiglu_codec_forward`)."""

    def __init__(self, codec, x, topk_ids, topk_weights, bank_tensors, out, workspace, stages=MOE_Q4_STAGE_ALL,
                 stream=None):
        self._keep = (x, topk_ids, topk_weights, tuple(bank_tensors), out, workspace)
        code, ptrs, (L, k, E, H, I) = _codec_args(codec, x, topk_ids, topk_weights, *bank_tensors)
        od = MOE_Q4_OUT_F32 if out.dtype == torch.float32 else MOE_Q4_OUT_BF16
        self._args = (code, *ptrs, L, k, E, H, I, _dev_ptr(out, (out.dtype,), "out"), od,
                      _dev_ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(), int(stages),
                      _stream_ptr(stream))
        self._fn = lib().moe_swiglu_codec_forward_stages

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st:
            raise MoeQ4Error(st, "moe_swiglu_codec_forward_stages")


def moe_q4_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement reference: one streaming read of ``buf`` (device tensor);
    ``sink`` is an int32 device tensor of at least 2 x CU-count words."""
    st = lib().moe_q4_stream_read(_dev_ptr(buf, (buf.dtype,), "buf"), buf.numel() * buf.element_size(),
                                  _dev_ptr(sink, _I32, "sink"), sink.numel(), _stream_ptr(stream))
    _check(st, "moe_q4_stream_read")
