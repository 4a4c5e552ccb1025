"""Thin Python binding of libmxfp4_moe.so (include/mxfp4_moe.h).

Argument marshalling only: each function checks dtypes, contiguity and
devices of the torch tensors it is given, then passes their device pointers,
the sizes and the current HIP stream to the C entry point of the same name.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes

import numpy as np
import os
from typing import Optional

import torch

MXFP4_OK = 0
MXFP4_PATH_AUTO, MXFP4_PATH_GEMV, MXFP4_PATH_GEMM = 0, 1, 2
MXFP4_ROUTE_ERR_ID_RANGE, MXFP4_ROUTE_ERR_ID_DUP = 1, 2
MXFP4_MAX_EXPERTS, MXFP4_MAX_TOPK = 512, 32
MXFP4_DECODE_MAX_EXPERTS, MXFP4_DECODE_MAX_K, MXFP4_GEMM_MAX_K = 64, 3072, 8192
MXFP4_NOALLOC_SCRATCH_BYTES = 128 << 20

#: the C entry points this binding uses (all declared in include/mxfp4_moe.h)
ENTRY_POINTS = (
    "mxfp4_status_string",
    "mxfp4_last_error",
    "mxfp4_moe_route_group",
    "mxfp4_expert_proj_workspace_size",
    "mxfp4_expert_proj",
    "mxfp4_expert_proj_swiglu",
    "moe_combine",
    "mxfp4_moe_decode",
    "mxfp4_dequantize",
    "mxfp4_moe_dense_route",
    "mxfp4_moe_router",
    "mxfp4_moe_decode_swiglu",
    "mxfp4_expert_proj_combine",
    "mxfp4_expert_proj_noalloc",
    "mxfp4_expert_proj_combine_routed",
    "mxfp4_moe_decode_batch",
    "mxfp4_moe_decode_batch_swiglu",
)

_lib_handle = None


def library_path() -> str:
    """The in-tree libmxfp4_moe.so, or the build named by MXFP4_MOE_LIB (the
    host-sanitizer build of the same sources, for the ABI tests)."""
    return os.environ.get("MXFP4_MOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libmxfp4_moe.so")


class MXFP4Error(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_text(status)} ({status}): {detail}")
        self.status = status


def load_library():
    """Load libmxfp4_moe.so and declare the C signatures (raises if it is not built)."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m mxfp4_mixture_experts_amd.build_lib`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mxfp4_status_string.argtypes = [i32]
    lib.mxfp4_status_string.restype = ctypes.c_char_p
    lib.mxfp4_last_error.argtypes = []
    lib.mxfp4_last_error.restype = ctypes.c_char_p
    lib.mxfp4_moe_route_group.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.mxfp4_moe_route_group.restype = i32
    lib.mxfp4_expert_proj_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.mxfp4_expert_proj_workspace_size.restype = sz
    lib.mxfp4_expert_proj.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.mxfp4_expert_proj_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, i32, vp]
    lib.mxfp4_expert_proj_noalloc.restype = i32
    lib.mxfp4_expert_proj.restype = i32
    lib.mxfp4_expert_proj_swiglu.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, i32, vp, sz, vp]
    lib.mxfp4_expert_proj_swiglu.restype = i32
    lib.moe_combine.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.moe_combine.restype = i32
    lib.mxfp4_moe_decode.argtypes = [vp, i32, i32, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    lib.mxfp4_moe_decode.restype = i32
    lib.mxfp4_dequantize.argtypes = [vp, vp, ctypes.c_longlong, i32, vp, vp]
    lib.mxfp4_dequantize.restype = i32
    lib.mxfp4_moe_dense_route.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.mxfp4_moe_dense_route.restype = i32
    lib.mxfp4_moe_router.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    lib.mxfp4_moe_router.restype = i32
    lib.mxfp4_moe_decode_swiglu.argtypes = [vp, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.mxfp4_moe_decode_swiglu.restype = i32
    lib.mxfp4_moe_decode_batch.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                           vp, vp]
    lib.mxfp4_moe_decode_batch.restype = i32
    lib.mxfp4_moe_decode_batch_swiglu.argtypes = [vp, i32, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp,
                                                  vp, vp]
    lib.mxfp4_moe_decode_batch_swiglu.restype = i32
    lib.mxfp4_expert_proj_combine.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.mxfp4_expert_proj_combine.restype = i32
    lib.mxfp4_expert_proj_combine_routed.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp,
                                                     vp, vp, i32, vp, sz, vp]
    lib.mxfp4_expert_proj_combine_routed.restype = i32
    _lib_handle = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().mxfp4_status_string(status).decode()
    except ImportError:
        return "status"


def _check(status: int):
    if status != MXFP4_OK:
        raise MXFP4Error(status, load_library().mxfp4_last_error().decode())


def _ptr(t: Optional[torch.Tensor], name: str, dtypes, device=None):
    if t is None:
        return None
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def mxfp4_moe_route_group(logits, ids_in, T: int, E: int, k: int, topk_ids, gates, expert_offsets,
                          sorted_rows, error_word=None, stream=None):
    """Route and group (mxfp4_moe_route_group).  logits [T,E] bf16 or None, ids_in [T,k] i32 or
    None; writes topk_ids [T,k] i32, gates [T,k] f32 (optional), expert_offsets [E+1] i32,
    sorted_rows [T*k] i32 and error_word [1] i32 (optional)."""
    lib = load_library()
    dev = expert_offsets.device
    st = lib.mxfp4_moe_route_group(
        _ptr(logits, "logits", _BF16, dev), _ptr(ids_in, "ids_in", _I32, dev), int(T), int(E), int(k),
        _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(error_word, "error_word", _I32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_expert_proj_workspace_size(E: int, N: int, T: int, k: int, K: int, x_per_slot: bool,
                                     path: int = MXFP4_PATH_AUTO) -> int:
    n = load_library().mxfp4_expert_proj_workspace_size(int(E), int(N), int(T), int(k), int(K),
                                                        int(bool(x_per_slot)), int(path))
    if n == ctypes.c_size_t(-1).value:
        raise MXFP4Error(1, "invalid sizes for the workspace query")
    return int(n)


def mxfp4_expert_proj(blocks, scales, bias, E: int, N: int, K: int, x, x_per_slot: bool, T: int, k: int,
                      expert_offsets, sorted_rows, out, path: int = MXFP4_PATH_AUTO, workspace=None,
                      stream=None):
    """The routed expert projection (mxfp4_expert_proj); out [T,k,N] f32 is written in place.
    workspace: a uint8 device tensor of at least mxfp4_expert_proj_workspace_size(...) bytes."""
    lib = load_library()
    dev = out.device
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace", _U8, dev)
        ws_bytes = workspace.numel()
    st = lib.mxfp4_expert_proj(
        _ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev),
        int(E), int(N), int(K), _ptr(x, "x", _BF16, dev), int(bool(x_per_slot)), int(T), int(k),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(out, "out", _F32, dev), int(path), ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream, dev))
    _check(st)


def mxfp4_expert_proj_noalloc(blocks, scales, bias, E: int, N: int, K: int, x, x_per_slot: bool, T: int, k: int,
                              expert_offsets, sorted_rows, out, path: int = MXFP4_PATH_AUTO, stream=None):
    """mxfp4_expert_proj with the library's static scratch instead of a workspace
    (mxfp4_expert_proj_noalloc); out [T,k,N] f32 is written in place."""
    lib = load_library()
    dev = out.device
    st = lib.mxfp4_expert_proj_noalloc(
        _ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev),
        int(E), int(N), int(K), _ptr(x, "x", _BF16, dev), int(bool(x_per_slot)), int(T), int(k),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(out, "out", _F32, dev), int(path), _stream(stream, dev))
    _check(st)


def mxfp4_expert_proj_swiglu(blocks, scales, bias, E: int, N: int, K: int, x, x_per_slot: bool, T: int, k: int,
                             expert_offsets, sorted_rows, act, path: int = MXFP4_PATH_AUTO, workspace=None,
                             stream=None):
    """The routed gate/up projection through the gated activation (mxfp4_expert_proj_swiglu);
    act [T,k,N/2] bf16 is written in place.  Workspace as for mxfp4_expert_proj."""
    lib = load_library()
    dev = act.device
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace", _U8, dev)
        ws_bytes = workspace.numel()
    st = lib.mxfp4_expert_proj_swiglu(
        _ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev),
        int(E), int(N), int(K), _ptr(x, "x", _BF16, dev), int(bool(x_per_slot)), int(T), int(k),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(act, "act", _BF16, dev), int(path), ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream, dev))
    _check(st)


def moe_combine(proj, gates, T: int, k: int, N: int, y, stream=None):
    """y[t,n] = sum_s gates[t,s] * proj[t,s,n] (moe_combine); y [T,N] f32 is overwritten."""
    lib = load_library()
    dev = y.device
    st = lib.moe_combine(_ptr(proj, "proj", _F32, dev), _ptr(gates, "gates", _F32, dev), int(T), int(k), int(N),
                         _ptr(y, "y", _F32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_decode(logits, E: int, k: int, blocks, scales, bias, N: int, K: int, x, x_per_slot: bool,
                     topk_ids, gates, expert_offsets, sorted_rows, out, error_word=None, stream=None):
    """One decode token in one launch (mxfp4_moe_decode): routing and grouping from logits [1,E]
    bf16 and the projection into out [1,k,N] f32, with the same outputs as
    mxfp4_moe_route_group followed by mxfp4_expert_proj."""
    lib = load_library()
    dev = out.device
    st = lib.mxfp4_moe_decode(
        _ptr(logits, "logits", _BF16, dev), int(E), int(k), _ptr(blocks, "blocks", _U8, dev),
        _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev), int(N), int(K), _ptr(x, "x", _BF16, dev),
        int(bool(x_per_slot)), _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(error_word, "error_word", _I32, dev), _ptr(out, "out", _F32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_decode_swiglu(logits, E: int, k: int, blocks, scales, bias, N: int, K: int, x, topk_ids, gates,
                            expert_offsets, sorted_rows, act, error_word=None, stream=None):
    """One decode token through the gate/up projection and the gated activation in one launch
    (mxfp4_moe_decode_swiglu): act [1,k,N/2] bf16, with the same outputs as
    mxfp4_moe_route_group followed by mxfp4_expert_proj_swiglu."""
    lib = load_library()
    dev = act.device
    st = lib.mxfp4_moe_decode_swiglu(
        _ptr(logits, "logits", _BF16, dev), int(E), int(k), _ptr(blocks, "blocks", _U8, dev),
        _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev), int(N), int(K), _ptr(x, "x", _BF16, dev),
        _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(error_word, "error_word", _I32, dev), _ptr(act, "act", _BF16, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_decode_batch(logits, T: int, E: int, k: int, blocks, scales, bias, N: int, K: int, x,
                           x_per_slot: bool, topk_ids, gates, expert_offsets, sorted_rows, out, error_word=None,
                           stream=None):
    """Up to 64 decode tokens in one launch (mxfp4_moe_decode_batch): routing and grouping from
    logits [T,E] bf16 and the projection into out [T,k,N] f32, with the same outputs as
    mxfp4_moe_route_group followed by mxfp4_expert_proj on the GEMV path."""
    lib = load_library()
    dev = out.device
    st = lib.mxfp4_moe_decode_batch(
        _ptr(logits, "logits", _BF16, dev), int(T), int(E), int(k), _ptr(blocks, "blocks", _U8, dev),
        _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev), int(N), int(K), _ptr(x, "x", _BF16, dev),
        int(bool(x_per_slot)), _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(error_word, "error_word", _I32, dev), _ptr(out, "out", _F32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_decode_batch_swiglu(logits, T: int, E: int, k: int, blocks, scales, bias, N: int, K: int, x,
                                  topk_ids, gates, expert_offsets, sorted_rows, act, error_word=None, stream=None):
    """Up to 64 decode tokens through the gate/up projection and the gated activation in one
    launch (mxfp4_moe_decode_batch_swiglu): act [T,k,N/2] bf16, with the same outputs as
    mxfp4_moe_route_group followed by mxfp4_expert_proj_swiglu on the GEMV path."""
    lib = load_library()
    dev = act.device
    st = lib.mxfp4_moe_decode_batch_swiglu(
        _ptr(logits, "logits", _BF16, dev), int(T), int(E), int(k), _ptr(blocks, "blocks", _U8, dev),
        _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev), int(N), int(K), _ptr(x, "x", _BF16, dev),
        _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(error_word, "error_word", _I32, dev), _ptr(act, "act", _BF16, dev), _stream(stream, dev))
    _check(st)


def mxfp4_dequantize(blocks, scales, out, stream=None):
    """MXFP4 -> bf16 (mxfp4_dequantize): blocks [..., KB, 16] u8 and scales [..., KB] u8 into
    out [..., KB * 32] bf16 (written in place), in the same layout."""
    lib = load_library()
    dev = out.device
    KB = int(blocks.shape[-2])
    if tuple(blocks.shape[:-1]) != tuple(scales.shape) or blocks.shape[-1] != 16:
        raise ValueError("blocks must be [..., KB, 16] and scales [..., KB]")
    if tuple(out.shape) != tuple(scales.shape[:-1]) + (KB * 32,):
        raise ValueError("out must be [..., KB * 32]")
    rows = int(np.prod(scales.shape[:-1])) if scales.dim() > 1 else 1
    st = lib.mxfp4_dequantize(_ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev),
                              ctypes.c_longlong(rows), KB * 32, _ptr(out, "out", _BF16, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_dense_route(logits, T: int, E: int, k: int, probs, stream=None):
    """Dense router weights (mxfp4_moe_dense_route): probs [T,E] f32, zero outside each token's top k."""
    lib = load_library()
    dev = probs.device
    st = lib.mxfp4_moe_dense_route(_ptr(logits, "logits", _BF16, dev), int(T), int(E), int(k),
                                   _ptr(probs, "probs", _F32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_moe_router(x, w, bias, T: int, H: int, E: int, logits, stream=None):
    """Router logits (mxfp4_moe_router): logits [T,E] bf16 = x [T,H] . w [E,H]^T + bias [E]."""
    lib = load_library()
    dev = logits.device
    st = lib.mxfp4_moe_router(_ptr(x, "x", _BF16, dev), _ptr(w, "w", _BF16, dev), _ptr(bias, "bias", _BF16, dev),
                              int(T), int(H), int(E), _ptr(logits, "logits", _BF16, dev), _stream(stream, dev))
    _check(st)


def mxfp4_expert_proj_combine(blocks, scales, bias, E: int, N: int, K: int, x, x_per_slot: bool, k: int, topk_ids,
                              gates, y, out=None, stream=None):
    """One token through its k experts and the gate-weighted combine in one launch
    (mxfp4_expert_proj_combine): y [1,N] f32 (and out [1,k,N] f32 if given), equal to
    mxfp4_expert_proj followed by moe_combine."""
    lib = load_library()
    dev = y.device
    st = lib.mxfp4_expert_proj_combine(
        _ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev), int(E),
        int(N), int(K), _ptr(x, "x", _BF16, dev), int(bool(x_per_slot)), int(k), _ptr(topk_ids, "topk_ids", _I32, dev),
        _ptr(gates, "gates", _F32, dev), _ptr(out, "out", _F32, dev), _ptr(y, "y", _F32, dev), _stream(stream, dev))
    _check(st)


def mxfp4_expert_proj_combine_routed(blocks, scales, bias, E: int, N: int, K: int, x, x_per_slot: bool, T: int,
                                     k: int, topk_ids, gates, expert_offsets, sorted_rows, out, y,
                                     path: int = MXFP4_PATH_AUTO, workspace=None, stream=None):
    """The routed projection of T tokens and the gate-weighted combine
    (mxfp4_expert_proj_combine_routed): out [T,k,N] f32 and y [T,N] f32, equal to
    mxfp4_expert_proj followed by moe_combine; the combine is fused into the
    grouped GEMM.  workspace: as for mxfp4_expert_proj."""
    lib = load_library()
    dev = y.device
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace", _U8, dev)
        ws_bytes = workspace.numel()
    st = lib.mxfp4_expert_proj_combine_routed(
        _ptr(blocks, "blocks", _U8, dev), _ptr(scales, "scales", _U8, dev), _ptr(bias, "bias", _BF16, dev),
        int(E), int(N), int(K), _ptr(x, "x", _BF16, dev), int(bool(x_per_slot)), int(T), int(k),
        _ptr(topk_ids, "topk_ids", _I32, dev), _ptr(gates, "gates", _F32, dev),
        _ptr(expert_offsets, "expert_offsets", _I32, dev), _ptr(sorted_rows, "sorted_rows", _I32, dev),
        _ptr(out, "out", _F32, dev), _ptr(y, "y", _F32, dev), int(path), ws_ptr, ctypes.c_size_t(ws_bytes),
        _stream(stream, dev))
    _check(st)
