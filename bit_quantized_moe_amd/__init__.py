"""Routed-expert MoE layer with low-bit (INT4 / 2-bit) experts on AMD MI355X.

Python binding of ``libbqmoe.so`` (declared in include/bqmoe.h).  The binding
only marshals arguments: it takes torch tensors for device memory, passes raw
pointers and the current HIP stream, and raises on a non-OK status.  Every
step of the layer runs in the library's HIP kernels; there is no fallback, so
a missing library is an error.

Tensor conventions: bf16 data as ``torch.bfloat16`` (or any 2-byte dtype
holding bf16 bits), packed code words as ``torch.int32`` (bit patterns of the
uint32 words), zero-points as ``torch.uint8``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

__all__ = [
    "MoEError", "lib", "route", "permute", "route_permute", "expert_ffn", "expert_table", "expert_ffn_table",
    "expert_ffn_nvfp4_table", "expert_ffn_nvfp4", "quant_act_nvfp4", "ffn_path",
    "layer", "layer_noalloc", "combine", "unpack_codes",
    "dequant_bf16", "Workspaces", "moe_layer", "LIB_PATH", "workspace_status", "set_wait_limit", "WS_WAIT_TIMEOUT",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbqmoe.so")

_c_int, _c_i64, _c_size, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "moe_abi_version": (_c_int, []),
    "moe_status_string": (ctypes.c_char_p, [_c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_status": (_c_int, [_vp, _c_size, _c_int, ctypes.POINTER(ctypes.c_uint32), _vp]),
    "moe_set_wait_limit": (_c_int, [_c_int]),
    "moe_route_workspace_size": (_c_size, [_c_int, _c_int]),
    "moe_route": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_permute_workspace_size": (_c_size, [_c_int, _c_int, _c_int]),
    "moe_permute": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_route_permute_workspace_size": (_c_size, [_c_int, _c_int, _c_int]),
    "moe_route_permute": (_c_int, [_vp, _vp, _vp] + [_c_int] * 4 + [_vp] * 7 + [_vp, _c_size, _vp]),
    "moe_expert_ffn_workspace_size": (_c_size, [_c_int] * 5),
    "moe_expert_ffn_path": (_c_int, [_c_int] * 7),
    "moe_expert_ffn_w4a16": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 5 + [_vp, _c_size, _vp]),
    "moe_expert_ffn_w2a16": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 7 + [_vp, _c_size, _vp]),
    "moe_expert_ffn_wna16": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 7 + [_vp] * 6 + [_vp, _vp, _c_size, _vp]),
    "moe_expert_ffn_nvfp4_workspace_size": (_c_size, [_c_int] * 5),
    "moe_expert_ffn_nvfp4": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [ctypes.c_float] * 2 + [_vp] * 6
                             + [_vp, _vp, _c_size, _vp]),
    "moe_quant_act_nvfp4": (_c_int, [_vp, _c_i64, ctypes.c_float, _vp, _vp, _vp]),
    "moe_expert_ffn_w4a16_table": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp, _vp, _c_size, _vp]),
    "moe_expert_ffn_w2a16_table": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [_vp, _vp, _vp, _c_size, _vp]),
    "moe_expert_ffn_wna16_table": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp, _c_size, _vp]),
    "moe_expert_ffn_nvfp4_table": (_c_int, [_vp, _vp, _vp, _vp] + [_c_int] * 5 + [ctypes.c_float] * 2
                                   + [_vp, _vp, _vp, _c_size, _vp]),
    "moe_device_address": (_c_int, [_vp, ctypes.POINTER(ctypes.c_uint64)]),
    "moe_combine": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "moe_layer_workspace_size": (_c_size, [_c_int] * 5),
    "moe_layer_w4a16": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 4 + [_vp] * 3 + [_vp, _c_size, _vp]),
    "moe_layer_nvfp4": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [ctypes.c_float] * 2 + [_vp] * 6 + [_vp] * 3
                        + [_vp, _c_size, _vp]),
    "moe_layer_wna16": (_c_int, [_vp, _vp, _vp] + [_c_int] * 7 + [_vp] * 6 + [_vp] * 3 + [_vp, _c_size, _vp]),
    "moe_layer_w2a16": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 6 + [_vp] * 3 + [_vp, _c_size, _vp]),
    "moe_layer_w4a16_noalloc": (_c_int, [_vp, _vp, _vp] + [_c_int] * 5 + [_vp] * 4 + [_vp] * 3 + [_vp]),
    "moe_unpack_codes": (_c_int, [_vp, _c_int, _c_i64, _vp, _vp]),
    "moe_probe_stream_blocks": (_c_size, [_c_size]),
    "moe_probe_stream_read": (_c_int, [_vp, _c_size, _vp, _vp]),
    "moe_probe_mfma": (_c_int, [_c_int, _c_int, _vp, _vp]),
    "moe_dequant_bf16": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "moe_dequant_bf16_grouped": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
}

_LIB: Optional[ctypes.CDLL] = None


class MoEError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libbqmoe.so (built by ``python -m bit_quantized_moe_amd.build``)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_moe_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, name: str) -> None:
    if status != 0:
        L = lib()
        raise MoEError(f"{name}: {L.moe_status_string(status).decode()} ({status}): {L.moe_last_error().decode()}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise MoEError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device):
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor) -> torch.device:
    if t.device.type != "cuda":
        raise MoEError("the MoE library runs on the GPU: pass device tensors")
    return t.device


WS_WAIT_TIMEOUT = 1  # MOE_WS_WAIT_TIMEOUT: a bounded cross-block wait gave up


def workspace_status(buf: torch.Tensor, clear: bool = True) -> int:
    """Sticky error flags of a workspace (moe_workspace_status; waits for the current stream)."""
    dev = _dev(buf)
    flags = ctypes.c_uint32(0)
    _check(lib().moe_workspace_status(_p(buf), buf.numel() * buf.element_size(), int(bool(clear)),
                                      ctypes.byref(flags), _stream(dev)), "moe_workspace_status")
    return int(flags.value)


def set_wait_limit(spins: int) -> int:
    """Polling rounds before a bounded wait gives up (a test hook; < 0 restores the default).  Returns the old limit."""
    return int(lib().moe_set_wait_limit(int(spins)))


# workspaces that start with a control block (the rest hold none)
_CTL_WORKSPACES = ("route", "ffn", "ffn_nvfp4", "layer")


class Workspaces:
    """Zero-initialised device workspaces, grown on demand and reused across calls.

    Each workspace starts with a control block that the kernels leave zeroed,
    so a buffer can be reused by consecutive calls on one stream.  check()
    reads the control blocks' error flags and raises if a wait timed out.
    """

    def __init__(self, device):
        self.device = torch.device(device)
        self._bufs: Dict[str, torch.Tensor] = {}

    def get(self, name: str, nbytes: int) -> torch.Tensor:
        b = self._bufs.get(name)
        if b is None or b.numel() < nbytes:
            b = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._bufs[name] = b
        return b

    def check(self) -> None:
        """Raise MoEError if a bounded wait of a call made with these workspaces
        gave up (its outputs are unreliable); the flags are cleared and the
        affected workspace zeroed, so the buffers can be used again."""
        bad = []
        for name, b in self._bufs.items():
            if name in _CTL_WORKSPACES and b.numel() >= 4096 and workspace_status(b, clear=True):
                b.zero_()
                bad.append(name)
        if bad:
            raise MoEError(f"a bounded wait timed out in the {', '.join(bad)} workspace(s): "
                           "the outputs of those calls are unreliable (workspaces zeroed)")


def route(x: torch.Tensor, w_router: torch.Tensor, k: int, logit_bias: Optional[torch.Tensor] = None,
          want_logits: bool = False, ws: Optional[Workspaces] = None):
    """Router logits, top-k ids (int32 [T, k]) and softmax gates (float32 [T, k])."""
    dev = _dev(x)
    T, H = x.shape
    E = w_router.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    L = lib()
    nbytes = L.moe_route_workspace_size(T, E)
    w = (ws or Workspaces(dev)).get("route", nbytes)
    _check(L.moe_route(_p(x), _p(w_router), _p(logit_bias), T, H, E, k, _p(ids), _p(gates), _p(logits),
                       _p(w), w.numel(), _stream(dev)), "moe_route")
    return (ids, gates, logits) if want_logits else (ids, gates)


def permute(ids: torch.Tensor, E: int, ws: Optional[Workspaces] = None):
    """Stable grouping of rows by expert: (offsets [E+1], sorted_rows, row_pos, active)."""
    dev = _dev(ids)
    T, k = ids.shape
    n = T * k
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_rows = torch.empty(n, dtype=torch.int32, device=dev)
    row_pos = torch.empty(n, dtype=torch.int32, device=dev)
    active = torch.empty(1 + min(E, n), dtype=torch.int32, device=dev)
    L = lib()
    nbytes = L.moe_permute_workspace_size(T, k, E)
    w = (ws or Workspaces(dev)).get("permute", nbytes) if nbytes else None
    _check(L.moe_permute(_p(ids), T, k, E, _p(offsets), _p(sorted_rows), _p(row_pos), _p(active), _p(w),
                         0 if w is None else w.numel(), _stream(dev)), "moe_permute")
    return offsets, sorted_rows, row_pos, active


def route_permute(x: torch.Tensor, w_router: torch.Tensor, k: int, logit_bias: Optional[torch.Tensor] = None,
                  want_logits: bool = False, ws: Optional[Workspaces] = None) -> Dict[str, torch.Tensor]:
    """route() then permute() in one library call (one launch for small batches).

    Returns ids, gates, offsets, sorted_rows, row_pos, active (and logits)."""
    dev = _dev(x)
    T, H = x.shape
    E = w_router.shape[0]
    n = T * k
    out = dict(
        ids=torch.empty((T, k), dtype=torch.int32, device=dev),
        gates=torch.empty((T, k), dtype=torch.float32, device=dev),
        offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
        sorted_rows=torch.empty(n, dtype=torch.int32, device=dev),
        row_pos=torch.empty(n, dtype=torch.int32, device=dev),
        active=torch.empty(1 + min(E, n), dtype=torch.int32, device=dev),
    )
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    L = lib()
    w = (ws or Workspaces(dev)).get("route", L.moe_route_permute_workspace_size(T, k, E))
    _check(L.moe_route_permute(_p(x), _p(w_router), _p(logit_bias), T, H, E, k, _p(out["ids"]), _p(out["gates"]),
                               _p(logits), _p(out["offsets"]), _p(out["sorted_rows"]), _p(out["row_pos"]),
                               _p(out["active"]), _p(w), w.numel(), _stream(dev)), "moe_route_permute")
    if want_logits:
        out["logits"] = logits
    return out


FFN_PATHS = {0: "decode", 1: "mid", 2: "gemm"}


def ffn_path(T: int, k: int, E: int, H: int, I: int, bits, group: int = 128) -> str:
    """The expert-FFN path ("decode", "mid" or "gemm") of these sizes and format
    (bits "nvfp4" for NVFP4)."""
    if bits == "nvfp4":
        bits, group = 4, 16
    p = lib().moe_expert_ffn_path(T, k, E, H, I, bits, group)
    if p < 0:
        raise MoEError(f"ffn_path: unsupported sizes or format ({bits} bits, group {group})")
    return FFN_PATHS[p]


def expert_ffn(x: torch.Tensor, offsets, sorted_rows, active, k: int, weights: Dict[str, torch.Tensor], bits: int,
               I: int, ws: Optional[Workspaces] = None, y_perm: Optional[torch.Tensor] = None,
               group: int = 128) -> torch.Tensor:
    """Per-expert gate_up -> SwiGLU -> down on the sorted rows; bf16 [T*k, H].

    bits 4 or 2 with group 128 call moe_expert_ffn_w4a16 / _w2a16; other
    formats (INT4 group 32, INT8 group 128 or 32, FP6 e2m3 with bits = 6)
    moe_expert_ffn_wna16."""
    dev = _dev(x)
    T, H = x.shape
    E = offsets.numel() - 1
    if y_perm is None:
        y_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    L = lib()
    nbytes = L.moe_expert_ffn_workspace_size(T, k, E, H, I)
    w = (ws or Workspaces(dev)).get("ffn", nbytes)
    st = _stream(dev)
    if bits not in (2, 4) or group != 128:
        s = L.moe_expert_ffn_wna16(_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I, bits, group,
                                   _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights.get("w13_zeros")),
                                   _p(weights["w2_codes"]), _p(weights["w2_scales"]), _p(weights.get("w2_zeros")),
                                   _p(y_perm), _p(w), w.numel(), st)
        _check(s, "moe_expert_ffn_wna16")
    elif bits == 4:
        s = L.moe_expert_ffn_w4a16(_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I,
                                   _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights["w2_codes"]),
                                   _p(weights["w2_scales"]), _p(y_perm), _p(w), w.numel(), st)
        _check(s, "moe_expert_ffn_w4a16")
    elif bits == 2:
        s = L.moe_expert_ffn_w2a16(_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I,
                                   _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights["w13_zeros"]),
                                   _p(weights["w2_codes"]), _p(weights["w2_scales"]), _p(weights["w2_zeros"]),
                                   _p(y_perm), _p(w), w.numel(), st)
        _check(s, "moe_expert_ffn_w2a16")
    else:
        raise MoEError("bits must be 2 or 4")
    return y_perm


_TABLE_FIELDS = ("w13_codes", "w13_scales", "w13_zeros", "w2_codes", "w2_scales", "w2_zeros")
# NVFP4 rows keep the address of each projection's float32 tensor scale where
# the other formats keep their zero-points
_TABLE_FIELDS_NVFP4 = ("w13_codes", "w13_scales", "w13_gscale", "w2_codes", "w2_scales", "w2_gscale")
_TABLE_ALIGN = {"codes": 16, "scales": 2, "zeros": 1, "gscale": 4}


def _device_address(L, ptr: int, what: str) -> int:
    a = ctypes.c_uint64(0)
    _check(L.moe_device_address(ctypes.c_void_p(ptr), ctypes.byref(a)), f"moe_device_address ({what})")
    return a.value


def expert_table(experts, bits, device=None) -> torch.Tensor:
    """Per-expert address table [E, 6] int64 for ``expert_ffn_table`` and
    ``expert_ffn_nvfp4_table``.

    ``experts`` is a list with one dict per expert (the keys of the stacked
    weights, each tensor that expert's own contiguous block, in device memory
    or in pinned host memory), or one stacked weights dict, whose [e] slices
    are used.  ``bits`` is the format's code width, or "nvfp4" (then entries 2
    and 5 hold the addresses of the expert's w13 / w2 float32 tensor scales).
    Zero-point entries are filled for 2-bit experts only.  Addresses go through
    ``moe_device_address``, which rejects memory the kernels cannot read; code
    blocks must be 16-byte, scale blocks 2-byte and tensor scales 4-byte
    aligned.  The table does not keep the expert tensors alive.  ``device`` is
    where the table itself lives: a CUDA device (default: the current one) or
    "pinned" for pinned host memory.
    """
    nv = bits == "nvfp4"
    fields = _TABLE_FIELDS_NVFP4 if nv else _TABLE_FIELDS
    if isinstance(experts, dict):
        E = experts["w13_codes"].shape[0]
        experts = [{n: t[e] for n, t in experts.items()} for e in range(E)]
    L = lib()
    rows = []
    for e, w in enumerate(experts):
        row = []
        for n in fields:
            kind = n.split("_", 1)[1]
            if kind == "zeros" and bits != 2:
                row.append(0)
                continue
            t = w.get(n)
            if t is None:
                raise MoEError(f"expert_table: expert {e} has no {n}")
            if not t.is_contiguous():
                raise MoEError(f"expert_table: expert {e} {n} is not contiguous")
            if t.data_ptr() % _TABLE_ALIGN[kind]:
                raise MoEError(f"expert_table: expert {e} {n} needs {_TABLE_ALIGN[kind]}-byte alignment")
            row.append(_device_address(L, t.data_ptr(), f"expert {e} {n}"))
        rows.append(row)
    tab = torch.tensor(rows, dtype=torch.int64).view(-1, len(fields))
    if device == "pinned":
        return tab.pin_memory()
    return tab.to(torch.device("cuda", torch.cuda.current_device()) if device is None else device)


def _table_arg(L, table: torch.Tensor, E: int, name: str) -> int:
    if table.dtype != torch.int64 or tuple(table.shape) != (E, len(_TABLE_FIELDS)):
        raise MoEError(f"{name}: table must be int64 [{E}, {len(_TABLE_FIELDS)}]")
    if not (table.is_cuda or table.is_pinned()):
        raise MoEError(f"{name}: the table must be in device or pinned host memory")
    return _p(table) if table.is_cuda else _device_address(L, _p(table), "table")


def expert_ffn_table(x: torch.Tensor, offsets, sorted_rows, active, k: int, table: torch.Tensor, bits: int, I: int,
                     ws: Optional[Workspaces] = None, y_perm: Optional[torch.Tensor] = None,
                     group: int = 128) -> torch.Tensor:
    """``expert_ffn`` with the expert weights found through an address table
    (bits 4 or 2 with group 128: the w4a16 / w2a16 table calls; other formats
    the wna16 table call)."""
    dev = _dev(x)
    T, H = x.shape
    E = offsets.numel() - 1
    L = lib()
    tab_ptr = _table_arg(L, table, E, "expert_ffn_table")
    if y_perm is None:
        y_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    nbytes = L.moe_expert_ffn_workspace_size(T, k, E, H, I)
    w = (ws or Workspaces(dev)).get("ffn", nbytes)
    common = (_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I)
    tail = (tab_ptr, _p(y_perm), _p(w), w.numel(), _stream(dev))
    if bits in (2, 4) and group == 128:
        name = "moe_expert_ffn_w4a16_table" if bits == 4 else "moe_expert_ffn_w2a16_table"
        s = getattr(L, name)(*common, *tail)
    else:
        name = "moe_expert_ffn_wna16_table"
        s = L.moe_expert_ffn_wna16_table(*common, bits, group, *tail)
    _check(s, name)
    return y_perm


def expert_ffn_nvfp4_table(x: torch.Tensor, offsets, sorted_rows, active, k: int, table: torch.Tensor, I: int,
                           x_gscale: float, h_gscale: float, ws: Optional[Workspaces] = None,
                           y_perm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``expert_ffn_nvfp4`` with the experts found through an address table
    (``expert_table(..., "nvfp4")``)."""
    dev = _dev(x)
    T, H = x.shape
    E = offsets.numel() - 1
    L = lib()
    tab_ptr = _table_arg(L, table, E, "expert_ffn_nvfp4_table")
    if y_perm is None:
        y_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    w = (ws or Workspaces(dev)).get("ffn_nvfp4", L.moe_expert_ffn_nvfp4_workspace_size(T, k, E, H, I))
    _check(L.moe_expert_ffn_nvfp4_table(_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I,
                                        float(x_gscale), float(h_gscale), tab_ptr, _p(y_perm), _p(w), w.numel(),
                                        _stream(dev)), "moe_expert_ffn_nvfp4_table")
    return y_perm


def quant_act_nvfp4(x: torch.Tensor, gscale: float, want_scales: bool = False):
    """NVFP4 activation quantiser: bf16 q * s of each value (and the E4M3 group-scale codes)."""
    dev = _dev(x)
    vals = torch.empty_like(x, dtype=torch.bfloat16)
    sc = torch.empty(x.numel() // 16, dtype=torch.uint8, device=dev) if want_scales else None
    _check(lib().moe_quant_act_nvfp4(_p(x), x.numel(), float(gscale), _p(vals), _p(sc), _stream(dev)),
           "moe_quant_act_nvfp4")
    return (vals, sc) if want_scales else vals


def expert_ffn_nvfp4(x: torch.Tensor, offsets, sorted_rows, active, k: int, weights: Dict[str, torch.Tensor], I: int,
                     x_gscale: float, h_gscale: float, ws: Optional[Workspaces] = None,
                     y_perm: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Expert FFN with NVFP4 W4A4 experts (weights: *_codes, *_scales (E4M3 uint8), *_gscale (float32 [E]))."""
    dev = _dev(x)
    T, H = x.shape
    E = offsets.numel() - 1
    if y_perm is None:
        y_perm = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    L = lib()
    w = (ws or Workspaces(dev)).get("ffn_nvfp4", L.moe_expert_ffn_nvfp4_workspace_size(T, k, E, H, I))
    _check(L.moe_expert_ffn_nvfp4(_p(x), _p(offsets), _p(sorted_rows), _p(active), T, k, E, H, I, float(x_gscale),
                                  float(h_gscale), _p(weights["w13_codes"]), _p(weights["w13_scales"]),
                                  _p(weights["w13_gscale"]), _p(weights["w2_codes"]), _p(weights["w2_scales"]),
                                  _p(weights["w2_gscale"]), _p(y_perm), _p(w), w.numel(), _stream(dev)),
           "moe_expert_ffn_nvfp4")
    return y_perm


def combine(y_perm: torch.Tensor, row_pos: torch.Tensor, gates: torch.Tensor) -> torch.Tensor:
    """Gate-weighted sum of each token's k expert rows; bf16 [T, H]."""
    dev = _dev(y_perm)
    T, k = gates.shape
    H = y_perm.shape[1]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _check(lib().moe_combine(_p(y_perm), _p(row_pos), _p(gates), T, k, H, _p(y), _stream(dev)), "moe_combine")
    return y


def layer(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor], weights: Dict[str, torch.Tensor],
          k: int, bits: int, I: int, ws: Optional[Workspaces] = None, want_routing: bool = False, group: int = 128):
    """The whole decode layer (T <= 16) in one library call; returns y (and ids, gates)."""
    dev = _dev(x)
    T, H = x.shape
    E = w_router.shape[0]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if want_routing else None
    gates = torch.empty((T, k), dtype=torch.float32, device=dev) if want_routing else None
    L = lib()
    w = (ws or Workspaces(dev)).get("layer", L.moe_layer_workspace_size(T, k, E, H, I))
    head = (_p(x), _p(w_router), _p(logit_bias), T, H, E, k, I)
    tail = (_p(y), _p(ids), _p(gates), _p(w), w.numel(), _stream(dev))
    if bits not in (2, 4) or group != 128:
        s = L.moe_layer_wna16(*head, bits, group, _p(weights["w13_codes"]), _p(weights["w13_scales"]),
                              _p(weights.get("w13_zeros")), _p(weights["w2_codes"]), _p(weights["w2_scales"]),
                              _p(weights.get("w2_zeros")), *tail)
        _check(s, "moe_layer_wna16")
        return (y, ids, gates) if want_routing else y
    if bits == 4:
        s = L.moe_layer_w4a16(*head, _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights["w2_codes"]),
                              _p(weights["w2_scales"]), *tail)
    elif bits == 2:
        s = L.moe_layer_w2a16(*head, _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights["w13_zeros"]),
                              _p(weights["w2_codes"]), _p(weights["w2_scales"]), _p(weights["w2_zeros"]), *tail)
    else:
        raise MoEError("bits must be 2 or 4")
    _check(s, f"moe_layer_w{bits}a16")
    return (y, ids, gates) if want_routing else y


def layer_noalloc(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor],
                  weights: Dict[str, torch.Tensor], k: int, I: int, y: Optional[torch.Tensor] = None,
                  ids: Optional[torch.Tensor] = None, gates: Optional[torch.Tensor] = None):
    """The INT4 one-launch layer with the library's own device scratch as its workspace
    (moe_layer_w4a16_noalloc): no workspace argument; outputs may be passed in preallocated."""
    dev = _dev(x)
    T, H = x.shape
    E = w_router.shape[0]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if y is None else y
    _check(lib().moe_layer_w4a16_noalloc(_p(x), _p(w_router), _p(logit_bias), T, H, E, k, I,
                                         _p(weights["w13_codes"]), _p(weights["w13_scales"]),
                                         _p(weights["w2_codes"]), _p(weights["w2_scales"]), _p(y), _p(ids),
                                         _p(gates), _stream(dev)), "moe_layer_w4a16_noalloc")
    return y


def layer_nvfp4(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor],
                weights: Dict[str, torch.Tensor], k: int, I: int, x_gscale: float, h_gscale: float,
                ws: Optional[Workspaces] = None, want_routing: bool = False):
    """The whole decode layer (T <= 16) with NVFP4 W4A4 experts in one library call."""
    dev = _dev(x)
    T, H = x.shape
    E = w_router.shape[0]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev) if want_routing else None
    gates = torch.empty((T, k), dtype=torch.float32, device=dev) if want_routing else None
    L = lib()
    w = (ws or Workspaces(dev)).get("layer", L.moe_layer_workspace_size(T, k, E, H, I))
    _check(L.moe_layer_nvfp4(_p(x), _p(w_router), _p(logit_bias), T, H, E, k, I, float(x_gscale), float(h_gscale),
                             _p(weights["w13_codes"]), _p(weights["w13_scales"]), _p(weights["w13_gscale"]),
                             _p(weights["w2_codes"]), _p(weights["w2_scales"]), _p(weights["w2_gscale"]), _p(y),
                             _p(ids), _p(gates), _p(w), w.numel(), _stream(dev)), "moe_layer_nvfp4")
    return (y, ids, gates) if want_routing else y


def unpack_codes(words: torch.Tensor, bits: int) -> torch.Tensor:
    """Signed codes of packed words (decode-path unpack routine); int8, K order (FP6: 8 * value)."""
    dev = _dev(words)
    n = words.numel()
    out = torch.empty(n * 32 // bits, dtype=torch.int8, device=dev)
    _check(lib().moe_unpack_codes(_p(words), bits, n, _p(out), _stream(dev)), "moe_unpack_codes")
    return out


def dequant_bf16(words: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor], bits: int,
                 N: int, K: int, group: int = 128) -> torch.Tensor:
    """[N, K] bf16 weights by the grouped-GEMM dequant routine."""
    dev = _dev(words)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    _check(lib().moe_dequant_bf16_grouped(_p(words), _p(scales), _p(zeros), bits, group, N, K, _p(out),
                                          _stream(dev)), "moe_dequant_bf16_grouped")
    return out


def moe_layer(x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor],
              weights: Dict[str, torch.Tensor], k: int, bits: int, I: int, ws: Optional[Workspaces] = None,
              want_logits: bool = False, group: int = 128) -> Dict[str, torch.Tensor]:
    """The whole layer: moe_route_permute, the expert FFN and moe_combine; returns every intermediate."""
    ws = ws or Workspaces(x.device)
    out = route_permute(x, w_router, k, logit_bias, want_logits=want_logits, ws=ws)
    y_perm = expert_ffn(x, out["offsets"], out["sorted_rows"], out["active"], k, weights, bits, I, ws=ws,
                        group=group)
    out["y_perm"] = y_perm
    out["y"] = combine(y_perm, out["row_pos"], out["gates"])
    return out
