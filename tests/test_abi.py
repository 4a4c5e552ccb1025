"""The C-ABI library loads, exports every symbol include/*.h declares, and rejects bad
arguments with the documented status before any HIP call.  No GPU needed."""
import ctypes
import glob
import os
import re

import pytest

from conftest import ROOT
from mxfp4_mixture_experts_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.library_path()), reason="library not built")


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const\s+char\s*\*|void)\s*\**\s*(\w+)\s*\(", src, re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert {"mxfp4_moe_route_group", "mxfp4_expert_proj", "moe_combine"} <= names
    assert set(B.ENTRY_POINTS) <= names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(B.library_path())
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = B.load_library()
    assert lib.mxfp4_status_string(0) == b"ok"
    assert b"gfx950" in lib.mxfp4_status_string(3)


def _route(lib, logits, ids, T, E, k, topk=1, off=1, rows=1):
    p = ctypes.c_void_p
    return lib.mxfp4_moe_route_group(logits and p(16), ids and p(16), T, E, k, topk and p(16), None,
                                     off and p(16), rows and p(16), None, None)


@pytest.mark.parametrize("args,why", [
    ((0, 0, 4, 32, 4), "no logits and no ids"),
    ((1, 0, -1, 32, 4), "negative T"),
    ((1, 0, 4, 0, 1), "E = 0"),
    ((1, 0, 4, 513, 4), "E above the limit"),
    ((1, 0, 4, 32, 0), "k = 0"),
    ((1, 0, 4, 4, 5), "k > E"),
    ((1, 0, 4, 64, 33), "k above the limit"),
])
def test_route_group_rejects_bad_arguments(args, why):
    lib = B.load_library()
    assert _route(lib, *args) == 1, why
    assert lib.mxfp4_last_error() != b""


def test_route_group_rejects_missing_outputs():
    lib = B.load_library()
    assert _route(lib, 1, 0, 4, 32, 4, off=0) == 1
    assert _route(lib, 1, 0, 4, 32, 4, rows=0) == 1


def _proj(lib, E=32, N=64, K=128, T=4, k=4, path=0, ws=None, ws_bytes=0, ptr=16, x_per_slot=0):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.mxfp4_expert_proj(p, p, None, E, N, K, p, x_per_slot, T, k, p, p, p, path,
                                 ws, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=100), 1), (dict(K=0), 1), (dict(N=0), 1), (dict(E=0), 1), (dict(k=33, E=64), 1),
    (dict(k=5, E=4), 1), (dict(T=-1), 1), (dict(path=7), 1), (dict(ptr=0), 1), (dict(ptr=8), 1),
    (dict(path=2, ws=None), 2), (dict(path=2, ws=ctypes.c_void_p(16), ws_bytes=10), 2),
    (dict(path=1, K=8192, T=64, k=4), 1),
    (dict(path=1, K=4128, T=64, k=4), 1),      # GEMV LDS staging: K <= 4096 when T > 4
    (dict(path=2, K=8224, ws=ctypes.c_void_p(16), ws_bytes=1 << 40), 1),  # GEMM: K <= 8192
    (dict(path=1, E=1, N=3_000_000, K=3072, T=64, k=1), 1),  # one expert's codes above 4 GiB (GEMV)
])
def test_expert_proj_rejects_bad_arguments(kw, status):
    lib = B.load_library()
    assert _proj(lib, **kw) == status


def _proj_swiglu(lib, E=32, N=64, K=128, T=4, k=4, path=0, ptr=16, act=16):
    p = ctypes.c_void_p(ptr) if ptr else None
    a = ctypes.c_void_p(act) if act else None
    return lib.mxfp4_expert_proj_swiglu(p, p, None, E, N, K, p, 0, T, k, p, p, a, path, None, ctypes.c_size_t(0),
                                        None)


@pytest.mark.parametrize("kw", [dict(N=63), dict(N=1), dict(act=0), dict(K=100), dict(E=0), dict(ptr=0),
                                dict(path=2)])
def test_expert_proj_swiglu_rejects_bad_arguments(kw):
    lib = B.load_library()
    assert _proj_swiglu(lib, **kw) in (1, 2), kw
    assert lib.mxfp4_last_error() != b""


def test_expert_proj_swiglu_t0_is_a_noop():
    lib = B.load_library()
    assert _proj_swiglu(lib, T=0, ptr=0, act=0) == 0


def _decode(lib, E=32, k=4, N=64, K=2880, ptr=16, logits=16):
    p = ctypes.c_void_p(ptr) if ptr else None
    lg = ctypes.c_void_p(logits) if logits else None
    return lib.mxfp4_moe_decode(lg, E, k, p, p, None, N, K, p, 0, p, None, p, p, None, p, None)


@pytest.mark.parametrize("kw", [
    dict(E=0), dict(E=65), dict(k=0), dict(k=5, E=4), dict(k=33, E=64), dict(N=0), dict(K=0), dict(K=100),
    dict(K=3104), dict(ptr=0), dict(ptr=8), dict(logits=0),
])
def test_moe_decode_rejects_bad_arguments(kw):
    lib = B.load_library()
    assert _decode(lib, **kw) == 1, kw
    assert lib.mxfp4_last_error() != b""


def _decode_swiglu(lib, E=32, k=4, N=64, K=2880, ptr=16, logits=16, act=16):
    p = ctypes.c_void_p(ptr) if ptr else None
    lg = ctypes.c_void_p(logits) if logits else None
    a = ctypes.c_void_p(act) if act else None
    return lib.mxfp4_moe_decode_swiglu(lg, E, k, p, p, None, N, K, p, p, None, p, p, None, a, None)


@pytest.mark.parametrize("kw", [
    dict(E=0), dict(E=65), dict(k=0), dict(k=5, E=4), dict(N=0), dict(N=63), dict(K=100), dict(K=3104),
    dict(ptr=0), dict(ptr=8), dict(logits=0), dict(act=0),
])
def test_moe_decode_swiglu_rejects_bad_arguments(kw):
    lib = B.load_library()
    assert _decode_swiglu(lib, **kw) == 1, kw
    assert lib.mxfp4_last_error() != b""


def _decode_batch(lib, T=64, E=32, k=4, N=64, K=2880, ptr=16, logits=16, out=16, swiglu=False):
    p = ctypes.c_void_p(ptr) if ptr else None
    lg = ctypes.c_void_p(logits) if logits else None
    o = ctypes.c_void_p(out) if out else None
    if swiglu:
        return lib.mxfp4_moe_decode_batch_swiglu(lg, T, E, k, p, p, None, N, K, p, p, None, p, p, None, o, None)
    return lib.mxfp4_moe_decode_batch(lg, T, E, k, p, p, None, N, K, p, 0, p, None, p, p, None, o, None)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("kw", [
    dict(T=0), dict(T=65), dict(E=0), dict(E=65), dict(k=0), dict(k=5, E=4), dict(k=33, E=64), dict(N=0),
    dict(K=0), dict(K=100), dict(K=3104), dict(ptr=0), dict(ptr=8), dict(logits=0), dict(out=0),
])
def test_moe_decode_batch_rejects_bad_arguments(kw, swiglu):
    lib = B.load_library()
    assert _decode_batch(lib, swiglu=swiglu, **kw) == 1, kw
    assert lib.mxfp4_last_error() != b""


def test_moe_decode_batch_rejects_experts_above_4gib():
    lib = B.load_library()
    assert _decode_batch(lib, T=2, E=1, k=1, N=3_000_000, K=3072) == 1
    assert b"4 GiB" in lib.mxfp4_last_error()


def test_moe_decode_batch_swiglu_needs_even_n():
    lib = B.load_library()
    assert _decode_batch(lib, N=63, swiglu=True) == 1
    assert b"even" in lib.mxfp4_last_error()


def test_expert_proj_t0_is_a_noop():
    lib = B.load_library()
    assert _proj(lib, T=0, ptr=0) == 0


def test_workspace_size():
    lib = B.load_library()
    ws = lib.mxfp4_expert_proj_workspace_size
    assert ws(32, 5760, 1, 4, 2880, 0, 1) == 0             # GEMV needs none
    assert ws(32, 5760, 1, 4, 2880, 0, 0) == 0             # auto: 4 rows over 4 experts -> GEMV
    assert ws(32, 2880, 64, 4, 2880, 1, 0) == 0            # auto: 256 rows over 32 experts -> GEMV
    # GEMM, K = 2880: 90 blocks = 45 MFMA k-steps, staged 8 blocks at a time:
    # 12 stages (padded to an even count), 48 k-steps.  The activations are
    # quantized into row tiles of 128 routed rows (at most ceil(R / 128) plus
    # one partial tile per expert); per tile, 32-row sub-tile and k-step (a
    # unit): 3 KB of codes for the two terms every block has, 3 KB for the third
    # and fourth terms of the units that take them, 256 bytes of scale words and
    # one byte with the unit's count of extra terms; the weight scales are
    # repacked to 2 KB per expert, 192-row panel (5760 rows = 30 panels) and
    # stage; the fused combine's arrival counters take 4 bytes per token and
    # panel.  Each region starts on a 256-byte boundary.
    al = lambda v: (v + 255) // 256 * 256

    def want(tiles, nkp, E, panels, stages, T):
        units = tiles * 4 * nkp
        return (al(units * 3072) * 2 + al(units * 256) + al(units) + al(E * panels * stages * 2048)
                + al(T * panels * 4))

    tiles = 16384 // 128 + 32
    assert ws(32, 5760, 4096, 4, 2880, 0, 2) == want(tiles, 48, 32, 30, 12, 4096)
    assert ws(32, 2880, 2048, 4, 2880, 1, 0) == want(64 + 32, 48, 32, 15, 12, 2048)
    # K = 64: one stage, padded to 2 (8 k-steps); 1024 rows over 8 experts: 8 + 8 tiles
    assert ws(8, 256, 512, 2, 64, 1, 2) == want(16, 8, 8, 2, 2, 512)
    # fewer rows than experts: at most one partial tile per row
    assert ws(32, 256, 3, 2, 64, 0, 2) == want(1 + 6, 8, 32, 2, 2, 3)
    assert ws(32, 5760, 4, 4, 100, 0, 0) == ctypes.c_size_t(-1).value
    assert ws(0, 5760, 4, 4, 128, 0, 0) == ctypes.c_size_t(-1).value
    assert ws(32, 0, 4, 4, 128, 0, 2) == ctypes.c_size_t(-1).value


def test_combine_rejects_bad_arguments():
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    assert lib.moe_combine(p, p, -1, 4, 8, p, None) == 1
    assert lib.moe_combine(p, p, 4, 0, 8, p, None) == 1
    assert lib.moe_combine(p, p, 4, 4, 0, p, None) == 1
    assert lib.moe_combine(None, p, 4, 4, 8, p, None) == 1
    assert lib.moe_combine(None, None, 0, 4, 8, None, None) == 0


def test_dequantize_rejects_bad_arguments():
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    assert lib.mxfp4_dequantize(p, p, ctypes.c_longlong(-1), 64, p, None) == 1
    assert lib.mxfp4_dequantize(p, p, ctypes.c_longlong(4), 100, p, None) == 1
    assert lib.mxfp4_dequantize(p, p, ctypes.c_longlong(4), 0, p, None) == 1
    assert lib.mxfp4_dequantize(None, p, ctypes.c_longlong(4), 64, p, None) == 1
    assert lib.mxfp4_dequantize(ctypes.c_void_p(8), p, ctypes.c_longlong(4), 64, p, None) == 1
    assert lib.mxfp4_dequantize(None, None, ctypes.c_longlong(0), 64, None, None) == 0


def test_dense_route_rejects_bad_arguments():
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    assert lib.mxfp4_moe_dense_route(p, -1, 32, 4, p, None) == 1
    assert lib.mxfp4_moe_dense_route(p, 4, 0, 1, p, None) == 1
    assert lib.mxfp4_moe_dense_route(p, 4, 513, 4, p, None) == 1
    assert lib.mxfp4_moe_dense_route(p, 4, 32, 33, p, None) == 1
    assert lib.mxfp4_moe_dense_route(None, 4, 32, 4, p, None) == 1
    assert lib.mxfp4_moe_dense_route(None, 0, 32, 4, None, None) == 0



def test_router_rejects_bad_arguments():
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    assert lib.mxfp4_moe_router(p, p, None, -1, 2880, 32, p, None) == 1
    assert lib.mxfp4_moe_router(p, p, None, 4, 100, 32, p, None) == 1   # H % 32 != 0
    assert lib.mxfp4_moe_router(p, p, None, 4, 0, 32, p, None) == 1
    assert lib.mxfp4_moe_router(p, p, None, 4, 2880, 0, p, None) == 1
    assert lib.mxfp4_moe_router(p, p, None, 4, 2880, 513, p, None) == 1
    assert lib.mxfp4_moe_router(None, p, None, 4, 2880, 32, p, None) == 1
    assert lib.mxfp4_moe_router(p, p, None, 4, 2880, 32, None, None) == 1
    assert lib.mxfp4_moe_router(ctypes.c_void_p(8), p, None, 4, 2880, 32, p, None) == 1  # x misaligned
    assert lib.mxfp4_last_error() != b""
    assert lib.mxfp4_moe_router(None, None, None, 0, 2880, 32, None, None) == 0


def test_proj_combine_rejects_bad_arguments():
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    f = lib.mxfp4_expert_proj_combine
    assert f(p, p, None, 0, 2880, 2880, p, 1, 4, p, p, None, p, None) == 1
    assert f(p, p, None, 32, 0, 2880, p, 1, 4, p, p, None, p, None) == 1
    assert f(p, p, None, 32, 2880, 3104, p, 1, 4, p, p, None, p, None) == 1   # K > MXFP4_DECODE_MAX_K
    assert f(p, p, None, 32, 2880, 100, p, 1, 4, p, p, None, p, None) == 1
    assert f(p, p, None, 4, 2880, 2880, p, 1, 5, p, p, None, p, None) == 1    # k > E
    assert f(p, p, None, 32, 2880, 2880, p, 1, 4, p, None, None, p, None) == 1  # no gates
    assert f(p, p, None, 32, 2880, 2880, p, 1, 4, p, p, None, None, None) == 1  # no y
    assert f(p, p, None, 32, 2880, 2880, ctypes.c_void_p(8), 1, 4, p, p, None, p, None) == 1  # x misaligned
    assert lib.mxfp4_last_error() != b""


def test_proj_combine_routed_rejects_bad_arguments():
    """mxfp4_expert_proj_combine_routed checks its arguments before any HIP call:
    the projection's checks, and the routing ids, gates, out and y it needs."""
    lib = B.load_library()
    p = ctypes.c_void_p(16)
    f = lib.mxfp4_expert_proj_combine_routed

    def call(E=32, N=2880, K=2880, x=p, T=64, k=4, ids=p, gates=p, out=p, y=p, path=1, ws=None, nbytes=0):
        return f(p, p, None, E, N, K, x, 1, T, k, ids, gates, p, p, out, y, path, ws, nbytes, None)

    assert call(E=0) == 1
    assert call(K=100) == 1
    assert call(k=33) == 1
    assert call(T=-1) == 1
    assert call(ids=None) == 1
    assert call(gates=None) == 1
    assert call(out=None) == 1
    assert call(y=None) == 1
    assert call(x=ctypes.c_void_p(8)) == 1
    assert call(T=1 << 16, N=5760, k=4) == 1                  # out past 4 GiB
    assert b"4 GiB" in lib.mxfp4_last_error()
    assert call(path=2) == 2                                  # the grouped GEMM needs its workspace
    assert b"workspace" in lib.mxfp4_last_error()
    assert call(T=0, ids=None, gates=None, out=None, y=None) == 0   # nothing to do


def test_noalloc_refuses_more_than_its_scratch():
    """mxfp4_expert_proj_noalloc rejects, before any HIP call, a problem whose grouped
    GEMM needs more than the static scratch (the gate_up prefill of 4096 tokens
    needs about 215 MB); the same problem on the GEMV path needs none."""
    lib = B.load_library()
    p = ctypes.c_void_p
    need = lib.mxfp4_expert_proj_workspace_size(32, 5760, 4096, 4, 2880, 0, 2)
    assert need > B.MXFP4_NOALLOC_SCRATCH_BYTES
    args = lambda T, path: (p(16), p(16), None, 32, 5760, 2880, p(16), 0, T, 4, p(16), p(16), p(16), path, None)
    assert lib.mxfp4_expert_proj_noalloc(*args(4096, 2)) == 2
    assert b"static scratch" in lib.mxfp4_last_error()
    small = lib.mxfp4_expert_proj_workspace_size(32, 5760, 512, 4, 2880, 0, 2)
    assert small <= B.MXFP4_NOALLOC_SCRATCH_BYTES
    assert lib.mxfp4_expert_proj_noalloc(*args(0, 2)) == 0           # T = 0: nothing to do
    assert lib.mxfp4_expert_proj_noalloc(p(16), p(16), None, 32, 5760, 2880, p(16), 0, 4, 4, p(16), p(16), None,
                                         2, None) == 1               # out is NULL
