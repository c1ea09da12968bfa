"""GPU parity of the further weight formats against the oracle.

INT4 symmetric with groups of 32 (the draft-layer experts of page
"Qwen3.8-Flash-Next on 2x RTX 3090", storage-format table) and INT8 symmetric
with groups of 128 or 32 (page "Qwen3.8-Flash-Next on one 24 GB GPU", "What
the patch does"; page "Qwen3.8-Flash-Next FP6-INT8", "Precision map" and
"Kernel-level verification"), and FP6 e2m3 with fp16 group-128 scales (same
page, opening paragraph and "Kernel-level verification"), through
moe_expert_ffn_wna16 on both FFN paths.
Bars as for the other formats: unpacked codes and dequantised bf16 values bit
for bit, outputs within 2e-2 relative Frobenius error (tensor-wide and per row).
"""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_amd as bq
import oracle
import workload
from gpu_util import bf16_np_to_f32, row_rel_err, to_dev, to_np, weights_to_dev

pytestmark = pytest.mark.gpu
TOL = 2e-2
FORMATS = [(4, 32), (8, 128), (8, 32), (6, 128)]
SIGMA = {4: 0.02, 8: 0.0015, 6: 0.02}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def test_unpack_int8_every_byte_every_position():
    words = []
    for pos in range(4):
        for v in range(256):
            w = 0
            for f in range(4):
                w |= (((v + 37 * f) % 256) if f != pos else v) << (8 * f)
            words.append(w)
    rng = np.random.default_rng(4)
    words = np.concatenate([np.array(words, np.uint32), rng.integers(0, 2**32, 1 << 18, dtype=np.uint32)])
    got = to_np(bq.unpack_codes(to_dev(words), 8))
    assert np.array_equal(got, oracle.unpack_codes(words, 8).ravel())


def test_unpack_fp6_every_code_every_position():
    """The decode routine's e2m3 conversion, as 8 * value: every code at every
    position of a 32-code group, then random words."""
    rows = []
    for pos in range(32):
        for c in range(64):
            stream = 0
            for f in range(32):
                stream |= ((c if f == pos else (c + 7 * f) % 64) << (6 * f))
            rows.append([(stream >> (32 * i)) & 0xFFFFFFFF for i in range(6)])
    rng = np.random.default_rng(6)
    words = np.concatenate([np.array(rows, np.uint32).ravel(), rng.integers(0, 2**32, 6 << 14, dtype=np.uint32)])
    got = to_np(bq.unpack_codes(to_dev(words), 6)).astype(np.int64)
    exp = (8 * oracle.e2m3_value(oracle.unpack_fp6_fields(words.reshape(-1, 6)).ravel())).astype(np.int64)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("bits,group", FORMATS)
def test_dequant_bf16_is_rounded_oracle(bits, group):
    rng = np.random.default_rng(5 + bits + group)
    N, K = 64, 1024
    words = rng.integers(0, 2**32, (N, K * bits // 32), dtype=np.uint32)
    if bits == 6:
        scales = (np.abs(rng.standard_normal((N, K // group))) * 0.03).astype(np.float16).view(np.uint16)
    else:
        scales = workload.bf16_bits(np.abs(rng.standard_normal((N, K // group))).astype(np.float32) * 0.03)
    got = to_np(bq.dequant_bf16(to_dev(words), to_dev(scales), None, bits, N, K, group=group))
    exp = workload.bf16_bits(oracle.dequantize(words, scales, None, bits, group))
    assert np.array_equal(got, exp)


def _check_ffn(inp, ws=None):
    sp = inp.spec
    wd = weights_to_dev(inp.weights)
    out = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), to_dev(inp.logit_bias) if inp.logit_bias is not None
                       else None, wd, sp.k, sp.bits, sp.I, ws=ws, group=sp.group)
    got = {kk: to_np(v) for kk, v in out.items()}
    ref = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, sp.bits, sp.I, group=sp.group)
    for key in ("ids", "offsets", "sorted_rows", "row_pos", "active"):
        assert np.array_equal(got[key], ref[key]), key
    yp, y = bf16_np_to_f32(got["y_perm"]), bf16_np_to_f32(got["y"])
    e1, e2 = oracle.rel_fro(yp, ref["y_perm"]), oracle.rel_fro(y, ref["y"])
    say(f"    T={sp.T} H={sp.H} I={sp.I} E={sp.E} k={sp.k}: y_perm rel-fro {e1:.2e}, y rel-fro {e2:.2e}")
    assert e1 <= TOL and e2 <= TOL
    assert np.max(row_rel_err(yp, ref["y_perm"])) <= TOL
    return got


@pytest.mark.parametrize("bits,group", FORMATS)
@pytest.mark.parametrize("T,H,I,E,k", [
    (1, 256, 128, 8, 2),        # decode, one token, ragged chunks
    (3, 512, 256, 16, 4),       # decode, a few tokens
    (16, 512, 256, 8, 4),       # decode, experts with more rows than one pass
    (40, 256, 128, 8, 2),       # grouped GEMM, ragged tiles
    (300, 1024, 256, 32, 4),    # grouped GEMM, several K and N tiles
], ids=lambda v: str(v))
def test_ffn_formats_small_shapes(bits, group, T, H, I, E, k):
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits, group=group,
                       scale_sigma=SIGMA[bits], seed=4000 + T + bits + group)
    _check_ffn(workload.make_layer_inputs(sp))


@pytest.mark.parametrize("bits,group", FORMATS)
def test_ffn_formats_full_chunk_decode_shapes(bits, group):
    """H = 4096, I = 1024: the decode kernel's full-chunk path (one token
    pipelined, and several tokens), and one workspace across calls."""
    ws = bq.Workspaces("cuda")
    for T, E, k in ((1, 8, 2), (1, 16, 8), (5, 8, 4), (16, 8, 4)):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=4096, I=1024, E=E, k=k, bits=bits, group=group,
                           scale_sigma=SIGMA[bits], seed=4100 + T + E + bits + group)
        _check_ffn(workload.make_layer_inputs(sp), ws=ws)
    torch.cuda.synchronize()
    for name, buf in ws._bufs.items():
        assert int(buf.view(torch.int32).abs().sum()) == 0, name


@pytest.mark.parametrize("name", ["decode_t1_h4096_e256_k8_i1024_int4g32", "decode_t1_h4096_e256_k8_i1024_int8",
                                  "decode_t1_h4096_e256_k8_i1024_int8g32", "decode_t1_h4096_e256_k8_i1024_fp6"])
def test_ffn_formats_decode_full_size(name):
    sp = workload.spec(name)
    _check_ffn(workload.make_layer_inputs(sp))


@pytest.mark.parametrize("name", ["prefill_t4096_h4096_e256_k8_i1024_int8g32", "prefill_t4096_h4096_e256_k8_i1024_fp6"])
def test_ffn_formats_prefill_full_size_sampled(name):
    sp = workload.spec(name)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    out = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), to_dev(inp.logit_bias), wd, sp.k, sp.bits, sp.I,
                       group=sp.group)
    got = {kk: to_np(v) for kk, v in out.items()}
    counts = np.diff(got["offsets"])
    act = got["active"][1:1 + got["active"][0]]
    by = sorted(act.tolist(), key=lambda e: counts[e])
    experts = [by[-1], by[len(by) // 2], by[0]]
    yp_ref = oracle.expert_ffn(inp.x, got["offsets"], got["sorted_rows"], sp.k, inp.weights, sp.bits, sp.I,
                               experts=experts, group=sp.group)
    yp = bf16_np_to_f32(got["y_perm"])
    for e in experts:
        o0, o1 = got["offsets"][e], got["offsets"][e + 1]
        err = oracle.rel_fro(yp[o0:o1], yp_ref[o0:o1])
        say(f"    expert {e} ({o1 - o0} rows): y_perm rel-fro {err:.2e}")
        assert err <= TOL
        assert np.max(row_rel_err(yp[o0:o1], yp_ref[o0:o1])) <= TOL


def test_wna16_matches_the_format_entry_points():
    """(4, 128) and (2, 128) through moe_expert_ffn_wna16 equal moe_expert_ffn_w4a16 / _w2a16 bit for bit."""
    for bits in (4, 2):
        for T in (1, 40):
            sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=512, I=256, E=16, k=4, bits=bits,
                               scale_sigma=0.02 if bits == 4 else 0.05, seed=4300 + T + bits)
            inp = workload.make_layer_inputs(sp)
            wd = weights_to_dev(inp.weights)
            r = bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), sp.k)
            args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"])
            a = bq.expert_ffn(*args, sp.k, wd, bits, sp.I)
            L = bq.lib()
            nbytes = L.moe_expert_ffn_workspace_size(T, sp.k, sp.E, sp.H, sp.I)
            w = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            b = torch.empty_like(a)
            st = torch.cuda.current_stream().cuda_stream
            s = L.moe_expert_ffn_wna16(args[0].data_ptr(), args[1].data_ptr(), args[2].data_ptr(), args[3].data_ptr(),
                                       T, sp.k, sp.E, sp.H, sp.I, bits, 128, wd["w13_codes"].data_ptr(),
                                       wd["w13_scales"].data_ptr(), wd["w13_zeros"].data_ptr() if bits == 2 else None,
                                       wd["w2_codes"].data_ptr(), wd["w2_scales"].data_ptr(),
                                       wd["w2_zeros"].data_ptr() if bits == 2 else None, b.data_ptr(), w.data_ptr(),
                                       nbytes, st)
            assert s == 0
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (bits, T)


def test_formats_alternate_on_one_workspace_and_route_edge_cases():
    """Every format on one set of workspaces, decode and GEMM paths in turn,
    including k = E (every expert active) and experts with no rows; the
    workspaces are all-zero at the end."""
    ws = bq.Workspaces("cuda")
    cases = [(4, 32, 1, 8, 8), (8, 128, 40, 8, 2), (6, 128, 3, 8, 8), (8, 32, 2, 16, 1), (4, 32, 300, 8, 2),
             (6, 128, 17, 32, 4), (2, 128, 1, 8, 8), (4, 128, 5, 16, 4)]
    for i, (bits, group, T, E, k) in enumerate(cases):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=512, I=256, E=E, k=k, bits=bits, group=group,
                           scale_sigma=SIGMA.get(bits, 0.05), seed=4400 + i)
        _check_ffn(workload.make_layer_inputs(sp), ws=ws)
    torch.cuda.synchronize()
    for name, buf in ws._bufs.items():
        assert int(buf.view(torch.int32).abs().sum()) == 0, name


@pytest.mark.parametrize("bits,group", [(4, 32), (8, 128), (8, 32), (6, 128)])
def test_one_launch_layer_formats_match_stages(bits, group):
    """moe_layer_wna16 (one launch) gives the stage calls' y, ids and gates bit for bit, and the oracle's y."""
    ws = bq.Workspaces("cuda")
    for T, H, I, E, k in ((1, 4096, 1024, 256, 8), (5, 512, 256, 16, 4), (16, 1024, 256, 32, 4)):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits, group=group,
                           scale_sigma=SIGMA[bits], seed=4600 + T + bits + group)
        inp = workload.make_layer_inputs(sp)
        wd = weights_to_dev(inp.weights)
        for rep in range(2):
            y, ids, gates = bq.layer(to_dev(inp.x), to_dev(inp.w_router), None, wd, sp.k, bits, sp.I, ws=ws,
                                     want_routing=True, group=group)
            st = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), None, wd, sp.k, bits, sp.I, ws=ws, group=group)
            assert torch.equal(ids, st["ids"]) and torch.equal(gates.view(torch.int32), st["gates"].view(torch.int32))
            assert torch.equal(y.view(torch.int16), st["y"].view(torch.int16)), (T, rep)
        ref = oracle.moe_layer(inp.x, inp.w_router, None, inp.weights, sp.k, bits, sp.I, group=group)
        err = oracle.rel_fro(bf16_np_to_f32(to_np(y)), ref["y"])
        say(f"    T={T} H={H}: one launch = stages bit for bit, y rel-fro {err:.2e}")
        assert err <= TOL
    torch.cuda.synchronize()
    for name, buf in ws._bufs.items():
        assert int(buf.view(torch.int32).abs().sum()) == 0, name
