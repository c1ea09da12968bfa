"""GPU: the expert FFN through a per-expert address table.

Each expert's weights sit in an allocation of their own (in device memory or in
pinned host memory, read in place), found through an int64 table (page
"Qwen3.8-Flash-Next on one 24 GB GPU", "What the patch does").  With the same
weights the table entry points must give the stacked-array entry points' y_perm
bit for bit, on the decode path (one token, a few tokens) and on the grouped
GEMM path, for every weight format (INT4 / 2-bit g128, INT4 g32, INT8 g128 and
g32, FP6 g128, NVFP4), and the array path is checked against the oracle
elsewhere; one small case per format is also checked against the oracle here.
"""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_amd as bq
import oracle
import workload
from gpu_util import bf16_np_to_f32, to_dev, to_np, weights_to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def _scattered_experts(wd, host_every=0):
    """One allocation per expert and tensor, made in reverse expert order; with
    host_every = n every n-th expert is copied to pinned host memory instead."""
    E = wd["w13_codes"].shape[0]
    experts = [None] * E
    for e in reversed(range(E)):
        on_host = host_every and e % host_every == 1
        experts[e] = {n: (t[e].cpu().pin_memory() if on_host else t[e].clone()) for n, t in wd.items()}
    return experts


def _route(inp, wd):
    sp = inp.spec
    bias = to_dev(inp.logit_bias) if inp.logit_bias is not None else None
    return bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), sp.k, bias)


CASES = [  # T, H, I, E, k: one token (full-chunk and ragged-chunk kernels), a few tokens, grouped GEMM
    (1, 4096, 1024, 16, 4),
    (1, 256, 128, 8, 2),
    (5, 512, 256, 16, 4),
    (16, 4096, 1024, 64, 8),
    (40, 256, 128, 8, 2),
    (300, 512, 256, 16, 4),
]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c)
@pytest.mark.parametrize("where", ["device", "mixed"])
def test_table_path_matches_arrays(bits, case, where):
    T, H, I, E, k = case
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=3100 + T + bits + E)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = _route(inp, wd)
    x = to_dev(inp.x)
    ref = bq.expert_ffn(x, r["offsets"], r["sorted_rows"], r["active"], k, wd, bits, I)
    experts = _scattered_experts(wd, host_every=3 if where == "mixed" else 0)
    table = bq.expert_table(experts, bits, device="pinned" if where == "mixed" else None)
    ws = bq.Workspaces("cuda")
    for rep in range(2):
        got = bq.expert_ffn_table(x, r["offsets"], r["sorted_rows"], r["active"], k, table, bits, I, ws=ws)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), rep
    torch.cuda.synchronize()
    assert int(ws._bufs["ffn"].view(torch.int32).abs().sum()) == 0
    say(f"    {where} experts, T={T}: table path bit-exact with the arrays")
    if T == 40 and where == "mixed":
        yp = oracle.expert_ffn(inp.x, to_np(r["offsets"]), to_np(r["sorted_rows"]), k, inp.weights, bits, I)
        assert oracle.rel_fro(bf16_np_to_f32(to_np(got)), yp) <= TOL


@pytest.mark.parametrize("bits", [4, 2])
def test_table_of_stacked_arrays_and_a_moved_expert(bits):
    """The table can point into the stacked arrays; rewriting two rows swaps two
    experts, which must equal the array path with those experts' weights swapped."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=3, H=512, I=256, E=8, k=8, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=3300 + bits)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = _route(inp, wd)
    x = to_dev(inp.x)
    args = (x, r["offsets"], r["sorted_rows"], r["active"], sp.k)
    table = bq.expert_table(wd, bits)
    got = bq.expert_ffn_table(*args, table, bits, sp.I)
    ref = bq.expert_ffn(*args, wd, bits, sp.I)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    perm = torch.arange(sp.E, device="cuda")
    perm[[2, 5]] = perm[[5, 2]]
    swapped = bq.expert_ffn_table(*args, table[perm].contiguous(), bits, sp.I)
    wd_sw = {n: t[perm].contiguous() for n, t in wd.items()}
    ref_sw = bq.expert_ffn(*args, wd_sw, bits, sp.I)
    assert torch.equal(swapped.view(torch.int16), ref_sw.view(torch.int16))
    assert not torch.equal(swapped.view(torch.int16), ref.view(torch.int16))


# every other format: INT4 g32, INT8 g128 / g32, FP6 e2m3 g128 through the wna16
# table call, and NVFP4 through its own
FORMATS = [(4, 32), (8, 128), (8, 32), (6, 128), ("nvfp4", 16)]
FORMAT_CASES = [  # T, H, I, E, k: one token on full chunks, a few tokens, grouped GEMM
    (1, 4096, 1024, 16, 4),
    (3, 512, 256, 16, 4),
    (40, 256, 128, 8, 2),
]


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: f"{f[0]}_g{f[1]}")
@pytest.mark.parametrize("case", FORMAT_CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d" % c)
@pytest.mark.parametrize("where", ["device", "mixed"])
def test_table_every_format_matches_arrays(fmt, case, where):
    bits, group = fmt
    nv = bits == "nvfp4"
    T, H, I, E, k = case
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=4 if nv else bits,
                       group=group, scale_sigma=0.02, seed=3500 + T + group + (0 if nv else bits))
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = _route(inp, wd)
    x = to_dev(inp.x)
    args = (x, r["offsets"], r["sorted_rows"], r["active"], k)
    if nv:
        ref = bq.expert_ffn_nvfp4(*args, wd, I, sp.nv_gx, sp.nv_gh)
    else:
        ref = bq.expert_ffn(*args, wd, bits, I, group=group)
    experts = _scattered_experts(wd, host_every=3 if where == "mixed" else 0)
    table = bq.expert_table(experts, bits, device="pinned" if where == "mixed" else None)
    ws = bq.Workspaces("cuda")
    for rep in range(2):
        if nv:
            got = bq.expert_ffn_nvfp4_table(*args, table, I, sp.nv_gx, sp.nv_gh, ws=ws)
        else:
            got = bq.expert_ffn_table(*args, table, bits, I, ws=ws, group=group)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), rep
    ws.check()
    say(f"    {fmt} {where} experts, T={T}: table path bit-exact with the arrays")
    if T == 40 and where == "mixed":
        off, srt = to_np(r["offsets"]), to_np(r["sorted_rows"])
        if nv:
            yp = oracle.expert_ffn_nvfp4(inp.x, off, srt, k, inp.weights, I, sp.nv_gx, sp.nv_gh)
        else:
            yp = oracle.expert_ffn(inp.x, off, srt, k, inp.weights, bits, I, group=group)
        assert oracle.rel_fro(bf16_np_to_f32(to_np(got)), yp) <= TOL


@pytest.mark.parametrize("bits", [4, 2])
def test_wna16_table_call_takes_the_g128_formats(bits):
    """moe_expert_ffn_wna16_table with bits 4 / 2 and group 128 equals the
    dedicated w4a16 / w2a16 table calls."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=5, H=512, I=256, E=16, k=4, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=3600 + bits)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = _route(inp, wd)
    x = to_dev(inp.x)
    table = bq.expert_table(wd, bits)
    ref = bq.expert_ffn_table(x, r["offsets"], r["sorted_rows"], r["active"], sp.k, table, bits, sp.I)
    L = bq.lib()
    T, H = x.shape
    nbytes = L.moe_expert_ffn_workspace_size(T, sp.k, sp.E, H, sp.I)
    w = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    got = torch.empty_like(ref)
    s = L.moe_expert_ffn_wna16_table(x.data_ptr(), r["offsets"].data_ptr(), r["sorted_rows"].data_ptr(),
                                     r["active"].data_ptr(), T, sp.k, sp.E, H, sp.I, bits, 128, table.data_ptr(),
                                     got.data_ptr(), w.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    assert s == 0, L.moe_last_error().decode()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    torch.cuda.synchronize()
    assert int(w.view(torch.int32).abs().sum()) == 0


def test_nvfp4_table_swaps_tensor_scales_with_the_expert():
    """Rewriting two NVFP4 rows swaps the experts' codes, group scales and
    tensor scales together: equal to the array path with those experts
    swapped in every array."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=3, H=512, I=256, E=8, k=8, bits=4, group=16, seed=3700)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    wd["w13_gscale"][5] *= 4.0                                   # make the swap visible in the tensor scales too
    r = _route(inp, wd)
    args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], sp.k)
    table = bq.expert_table(wd, "nvfp4")
    perm = torch.arange(sp.E, device="cuda")
    perm[[2, 5]] = perm[[5, 2]]
    got = bq.expert_ffn_nvfp4_table(*args, table[perm].contiguous(), sp.I, sp.nv_gx, sp.nv_gh)
    wd_sw = {n: t[perm].contiguous() for n, t in wd.items()}
    ref = bq.expert_ffn_nvfp4(*args, wd_sw, sp.I, sp.nv_gx, sp.nv_gh)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_table_rejects_pageable_host_memory_and_bad_tables():
    w = {"w13_codes": torch.zeros((4, 2), dtype=torch.int32)}          # pageable host memory
    with pytest.raises(bq.MoEError, match="device-readable|knows"):
        bq.expert_table([w], 4)
    x = torch.zeros((1, 256), dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(9, dtype=torch.int32, device="cuda")
    with pytest.raises(bq.MoEError, match="int64"):
        bq.expert_ffn_table(x, z, z[:1], z[:1], 1, torch.zeros((8, 5), dtype=torch.int64, device="cuda"), 4, 128)
    with pytest.raises(bq.MoEError, match="int64"):
        bq.expert_ffn_nvfp4_table(x, z, z[:1], z[:1], 1, torch.zeros((8, 6), dtype=torch.int32, device="cuda"),
                                  128, 1.0, 1.0)
    w = {"w13_codes": torch.zeros((4, 2), dtype=torch.int32, device="cuda")}
    with pytest.raises(bq.MoEError, match="no w13_gscale|no w13_scales"):
        bq.expert_table([w], "nvfp4")
    with pytest.raises(bq.MoEError, match="alignment"):
        bq.expert_table([{"w13_codes": torch.zeros(9, dtype=torch.int32, device="cuda")[1:]}], 4)
