"""The C ABI on the host: the library loads, exports what include/bqmoe.h declares,
and rejects bad arguments before touching the GPU (these run without a GPU)."""
import ctypes
import os
import re

import pytest

import bit_quantized_moe_amd as bq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "bqmoe.h")

OK, INVALID, SHAPE, MISALIGNED, WS_SMALL, HIP = range(6)
A = 1 << 20          # a fake, well-aligned device address: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = bq.lib()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(bq._SIGS)


def test_abi_version_and_status_strings():
    L = bq.lib()
    assert L.moe_abi_version() == 2
    for s in range(6):
        assert L.moe_status_string(s)
    assert L.moe_status_string(99) == b"unknown status"


def _route(T=4, H=256, E=8, k=2, x=A, w=A, ids=A, g=A, ws=A, wsb=1 << 20, bias=None, logits=None):
    return bq.lib().moe_route(x, w, bias, T, H, E, k, ids, g, logits, ws, wsb, None)


def test_route_argument_errors():
    L = bq.lib()
    assert _route(T=-1) == INVALID
    assert _route(k=0) == INVALID
    assert _route(k=9) == INVALID                 # k > E
    assert _route(E=8, k=33) == INVALID
    assert _route(E=2000) == SHAPE
    assert _route(H=200) == SHAPE                 # not a multiple of 128
    assert _route(x=None) == INVALID
    assert b"required" in L.moe_last_error()
    assert _route(x=A + 4) == MISALIGNED
    assert _route(ws=A + 128) == MISALIGNED
    assert _route(wsb=16) == WS_SMALL
    assert b"workspace" in L.moe_last_error()
    assert _route(T=0) == OK                      # empty batch: checked, nothing enqueued


def test_route_workspace_size():
    L = bq.lib()
    assert L.moe_route_workspace_size(1, 256) >= 4096 + 256 * 8     # control block + tagged logits
    assert L.moe_route_workspace_size(1, 256) % 256 == 0
    assert L.moe_route_workspace_size(-1, 8) == 0


def test_permute_argument_errors():
    L = bq.lib()
    f = lambda T=4, k=2, E=8, ids=A, off=A, sr=A, rp=A, act=A: L.moe_permute(ids, T, k, E, off, sr, rp, act, None, 0, None)
    assert f(T=-2) == INVALID
    assert f(k=0) == INVALID
    assert f(E=0) == SHAPE
    assert f(ids=None) == INVALID
    assert f(off=A + 2) == MISALIGNED
    assert f(T=0) == OK


def test_route_permute_argument_errors():
    L = bq.lib()

    def f(T=4, H=256, E=8, k=2, x=A, ids=A, off=A, act=A, ws=A, wsb=1 << 20):
        return L.moe_route_permute(x, A, None, T, H, E, k, ids, A, None, off, A, A, act, ws, wsb, None)
    assert f(T=-1) == INVALID
    assert f(k=9) == INVALID                      # k > E
    assert f(E=2000) == SHAPE
    assert f(H=200) == SHAPE
    assert f(x=None) == INVALID
    assert f(off=None) == INVALID                 # the permutation outputs are required
    assert f(act=A + 2) == MISALIGNED
    assert f(ws=A + 128) == MISALIGNED
    assert f(wsb=16) == WS_SMALL
    assert f(T=0) == OK
    # the workspace covers both the router's and the grouping's needs
    for T, k, E in [(1, 8, 256), (16, 8, 256), (4096, 8, 256), (33, 32, 1024)]:
        need = L.moe_route_permute_workspace_size(T, k, E)
        assert need % 256 == 0
        assert need >= L.moe_route_workspace_size(T, E) and need >= L.moe_permute_workspace_size(T, k, E)


def _ffn(bits=4, T=2, k=2, E=8, H=256, I=128, x=A, codes=A, ws=A, wsb=1 << 24, zeros=A):
    L = bq.lib()
    if bits == 4:
        return L.moe_expert_ffn_w4a16(x, A, A, A, T, k, E, H, I, codes, A, codes, A, A, ws, wsb, None)
    return L.moe_expert_ffn_w2a16(x, A, A, A, T, k, E, H, I, codes, A, zeros, codes, A, zeros, A, ws, wsb, None)


def test_ffn_argument_errors():
    L = bq.lib()
    assert _ffn(I=100) == SHAPE
    assert _ffn(H=64) == SHAPE
    assert _ffn(k=3, E=2) == INVALID
    assert _ffn(x=None) == INVALID
    assert _ffn(bits=2, zeros=None) == INVALID
    assert _ffn(codes=A + 8) == MISALIGNED
    assert _ffn(wsb=100) == WS_SMALL
    assert _ffn(T=0) == OK
    need = L.moe_expert_ffn_workspace_size(16, 8, 256, 4096, 1024)
    assert need >= 4096 + 16 * 8 * 1024 * 2 and need % 256 == 0


def _ffn_table(bits=4, T=2, k=2, E=8, H=256, I=128, x=A, tab=A, ws=A, wsb=1 << 24, group=128):
    L = bq.lib()
    if bits == "nvfp4":
        return L.moe_expert_ffn_nvfp4_table(x, A, A, A, T, k, E, H, I, 1.0, 1.0, tab, A, ws, wsb, None)
    if group != 128 or bits not in (2, 4):
        return L.moe_expert_ffn_wna16_table(x, A, A, A, T, k, E, H, I, bits, group, tab, A, ws, wsb, None)
    fn = L.moe_expert_ffn_w4a16_table if bits == 4 else L.moe_expert_ffn_w2a16_table
    return fn(x, A, A, A, T, k, E, H, I, tab, A, ws, wsb, None)


@pytest.mark.parametrize("bits", [4, 2, 8, 6, "nvfp4"])
def test_ffn_table_argument_errors(bits):
    assert _ffn_table(bits, tab=None) == INVALID
    assert _ffn_table(bits, tab=A + 4) == MISALIGNED
    assert _ffn_table(bits, I=100) == SHAPE
    assert _ffn_table(bits, x=None) == INVALID
    assert _ffn_table(bits, x=A + 8) == MISALIGNED
    assert _ffn_table(bits, wsb=100) == WS_SMALL
    assert _ffn_table(bits, T=0) == OK        # no weight arrays are needed beside the table


def test_ffn_table_format_and_scale_errors():
    L = bq.lib()
    assert _ffn_table(4, group=32, T=0) == OK
    assert _ffn_table(8, group=32, T=0) == OK
    for bits, group in ((2, 32), (6, 32), (4, 64), (3, 128), (4, 16)):
        assert _ffn_table(bits, group=group) == INVALID, (bits, group)
        assert "unsupported format" in L.moe_last_error().decode()
    for gx, gh in ((0.0, 1.0), (1.0, -1.0), (float("nan"), 1.0), (1.0, float("inf"))):
        assert L.moe_expert_ffn_nvfp4_table(A, A, A, A, 2, 2, 8, 256, 128, gx, gh, A, A, A, 1 << 24, None) == INVALID


def test_ffn_wna16_format_errors():
    L = bq.lib()
    f = lambda bits, g, **kw: L.moe_expert_ffn_wna16(A, A, A, A, 2, 2, 8, 256, 128, bits, g, A, A, kw.get("z", A), A,
                                                      A, kw.get("z", A), A, A, 1 << 24, None)
    assert f(4, 64) == INVALID and f(2, 32) == INVALID and f(3, 128) == INVALID and f(8, 16) == INVALID
    assert f(2, 128, z=None) == INVALID            # 2-bit needs zero-points
    for bits, g in ((4, 32), (8, 128), (8, 32)):
        assert L.moe_expert_ffn_wna16(A, A, A, A, 0, 2, 8, 256, 128, bits, g, A, A, None, A, A, None, A, A, 1 << 24,
                                      None) == OK
    assert L.moe_unpack_codes(A, 8, 0, A, None) == OK
    assert L.moe_dequant_bf16_grouped(A, A, None, 2, 32, 4, 128, A, None) == SHAPE
    assert L.moe_dequant_bf16_grouped(A, A, None, 8, 32, 0, 128, A, None) == OK


def _nv(T=2, k=2, E=8, H=256, I=128, gx=0.01, gh=0.01, x=A, codes=A, sc=A, g=A, ws=A, wsb=1 << 24):
    L = bq.lib()
    return L.moe_expert_ffn_nvfp4(x, A, A, A, T, k, E, H, I, gx, gh, codes, sc, g, codes, sc, g, A, ws, wsb, None)


def test_nvfp4_argument_errors():
    L = bq.lib()
    assert _nv(I=100) == SHAPE
    assert _nv(x=None) == INVALID and _nv(g=None) == INVALID and _nv(sc=None) == INVALID
    assert _nv(gx=0.0) == INVALID and _nv(gh=-1.0) == INVALID and _nv(gx=float("inf")) == INVALID
    assert _nv(gh=float("nan")) == INVALID
    assert _nv(codes=A + 8) == MISALIGNED and _nv(sc=A + 1) == MISALIGNED
    assert _nv(wsb=100) == WS_SMALL
    assert _nv(T=0) == OK
    need = L.moe_expert_ffn_nvfp4_workspace_size(16, 8, 256, 4096, 1024)
    assert need >= L.moe_expert_ffn_workspace_size(16, 8, 256, 4096, 1024) + 16 * 4096 * 2 and need % 256 == 0
    q = L.moe_quant_act_nvfp4
    assert q(A, 17, 0.1, A, None, None) == SHAPE
    assert q(None, 16, 0.1, A, None, None) == INVALID
    assert q(A, 16, 0.0, A, None, None) == INVALID
    assert q(A + 8, 16, 0.1, A, None, None) == MISALIGNED
    assert q(A, 0, 0.1, A, None, None) == OK


def test_device_address_argument_errors():
    L = bq.lib()
    out = ctypes.c_uint64(0)
    assert L.moe_device_address(None, ctypes.byref(out)) == INVALID
    assert L.moe_device_address(A, None) == INVALID


def test_combine_unpack_dequant_argument_errors():
    L = bq.lib()
    assert L.moe_combine(A, A, A, 4, 2, 100, A, None) == SHAPE       # H % 8
    assert L.moe_combine(None, A, A, 4, 2, 128, A, None) == INVALID
    assert L.moe_combine(A + 8, A, A, 4, 2, 128, A, None) == MISALIGNED
    assert L.moe_combine(A, A, A, 0, 2, 128, A, None) == OK
    assert L.moe_unpack_codes(A, 3, 10, A, None) == SHAPE
    assert L.moe_unpack_codes(A, 4, -1, A, None) == INVALID
    assert L.moe_unpack_codes(A, 4, 0, A, None) == OK
    assert L.moe_dequant_bf16(A, A, None, 2, 4, 128, A, None) == INVALID  # 2-bit needs zeros
    assert L.moe_dequant_bf16(A, A, None, 4, 4, 100, A, None) == SHAPE
    assert L.moe_dequant_bf16(A, A, None, 4, 0, 128, A, None) == OK


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(bq.MoEError):
        bq.route(torch.zeros((1, 256), dtype=torch.bfloat16), torch.zeros((8, 256), dtype=torch.bfloat16), 2)


def test_workspace_status_argument_errors():
    L = bq.lib()
    flags = ctypes.c_uint32(7)
    assert L.moe_workspace_status(None, 4096, 1, ctypes.byref(flags), None) == INVALID
    assert L.moe_workspace_status(A, 4096, 1, None, None) == INVALID
    assert L.moe_workspace_status(A + 16, 4096, 1, ctypes.byref(flags), None) == MISALIGNED
    assert L.moe_workspace_status(A, 1024, 1, ctypes.byref(flags), None) == WS_SMALL
    assert b"control block" in L.moe_last_error()
    assert flags.value == 7                            # untouched on an error


def test_wait_limit_set_and_restored():
    L = bq.lib()
    prev = L.moe_set_wait_limit(5)
    try:
        assert prev == 1 << 22
        assert L.moe_set_wait_limit(-1) == 5           # < 0 restores the default
        assert L.moe_set_wait_limit(-1) == 1 << 22
    finally:
        L.moe_set_wait_limit(-1)


def test_layer_noalloc_argument_errors():
    """Argument errors come back before the library looks up its scratch (no GPU needed)."""
    L = bq.lib()
    f = L.moe_layer_w4a16_noalloc
    args = [A, A, None, 1, 4096, 256, 8, 1024, A, A, A, A, A, None, None, None]
    assert f(*args[:3], 0, *args[4:]) == OK                          # T = 0: nothing to do
    bad = list(args); bad[0] = None
    assert f(*bad) == INVALID
    bad = list(args); bad[0] = A + 4
    assert f(*bad) == MISALIGNED
    bad = list(args); bad[3] = 16; bad[6] = 16                       # T*k = 256 at I = 4096: > 8 MiB
    bad[7] = 4096
    assert f(*bad) == SHAPE
    assert b"scratch" in L.moe_last_error()
    bad = list(args); bad[3] = 17                                    # one-launch layer: T <= 16
    assert f(*bad) == SHAPE


def test_expert_ffn_path_rule():
    """Host-side dispatch: decode up to about six rows per expert, the mid
    path up to 24 (INT4 / 2-bit g128, H and I multiples of 256), the grouped
    GEMMs beyond and for every other format."""
    L = bq.lib()
    f = L.moe_expert_ffn_path
    full = (4096, 1024)
    assert f(1, 8, 256, *full, 4, 128) == 0
    assert f(192, 8, 256, *full, 4, 128) == 0
    assert f(193, 8, 256, *full, 4, 128) == 1
    assert f(256, 8, 256, *full, 2, 128) == 1
    assert f(768, 8, 256, *full, 4, 128) == 1
    assert f(769, 8, 256, *full, 4, 128) == 2
    assert f(4096, 8, 256, *full, 4, 128) == 2
    assert f(256, 8, 256, *full, 8, 128) == 2 and f(256, 8, 256, *full, 4, 32) == 2
    assert f(256, 8, 256, *full, 6, 128) == 2 and f(256, 8, 256, *full, 4, 16) == 2
    assert f(1, 8, 256, *full, 4, 16) == 0
    assert f(40, 2, 8, 256, 128, 4, 128) == 2          # I not a multiple of 256
    assert f(40, 2, 8, 384, 256, 4, 128) == 2          # H not a multiple of 256
    assert f(40, 2, 8, 512, 512, 4, 128) == 1 and f(40, 2, 8, 256, 256, 2, 128) == 1
    assert f(0, 2, 8, 512, 512, 4, 128) == 0
    assert f(-1, 8, 256, *full, 4, 128) == -1 and f(1, 8, 256, *full, 3, 128) == -1
    assert bq.ffn_path(256, 8, 256, *full, 4) == "mid" and bq.ffn_path(1, 8, 256, *full, "nvfp4") == "decode"


def test_binding_exports_every_public_name():
    """Every name in the package's __all__ is defined."""
    assert [n for n in bq.__all__ if not hasattr(bq, n)] == []
    assert callable(bq.quant_act_nvfp4) and callable(bq.expert_ffn_nvfp4_table) and callable(bq.ffn_path)
