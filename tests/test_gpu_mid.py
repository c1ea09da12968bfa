"""GPU: the middle-batch expert FFN (between the decode kernel and the grouped GEMMs).

For each case the shape is first checked to take the mid path
(moe_expert_ffn_path); then y_perm of the INT4 and 2-bit calls is compared with
the float32 oracle (relative Frobenius error and every row within 2e-2), on the
GPU's own permutation (which is bit-exact with the oracle's elsewhere).  The
cases cover one and two 16-row tiles, ragged row counts, experts with more
than 32 rows (several passes over the weights, skewed routing), empty
experts, the address table, repeated calls on one workspace (bit-identical,
workspace left zero) and the full-size configurations of 256 and 512 tokens
(H = 4096, E = 256, top-8, I = 1024) on sampled experts.
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"[gpu-test] start {request.node.name}")
    yield
    torch.cuda.synchronize()


def _inputs(T, H, I, E, k, bits, seed, zipf=0.0):
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=seed, zipf_s=zipf)
    assert bq.ffn_path(T, k, E, H, I, bits) == "mid", (T, k, E, H, I, bits)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    bias = to_dev(inp.logit_bias) if inp.logit_bias is not None else None
    r = bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), k, bias)
    return sp, inp, wd, r


def _check(sp, inp, r, got, experts=None):
    off, srt = to_np(r["offsets"]), to_np(r["sorted_rows"])
    ref = oracle.expert_ffn(inp.x, off, srt, sp.k, inp.weights, sp.bits, sp.I, experts=experts)
    yp = bf16_np_to_f32(to_np(got))
    if experts is None:
        experts = [e for e in range(sp.E) if off[e + 1] > off[e]]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    err = oracle.rel_fro(yp[rows], ref[rows])
    worst = row_rel_err(yp[rows], ref[rows]).max()
    counts = np.diff(off)
    say(f"    T={sp.T} bits={sp.bits}: rows/expert max {counts.max()}, rel-fro {err:.2e}, worst row {worst:.2e}")
    assert err <= TOL and worst <= TOL
    return counts


CASES = [  # T, H, I, E, k, zipf: rows per expert ~10 (one tile), ~20 (two tiles), skewed (several passes)
    (40, 512, 512, 8, 2, 0.0),
    (40, 256, 256, 8, 2, 0.0),
    (90, 512, 1024, 8, 2, 0.0),
    (120, 1024, 512, 16, 3, 1.2),
    (70, 2048, 512, 32, 8, 0.0),
]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d_H%d_I%d_E%d_k%d_z%.1f" % c)
def test_mid_matches_oracle(bits, case):
    T, H, I, E, k, zipf = case
    sp, inp, wd, r = _inputs(T, H, I, E, k, bits, 4100 + T + bits, zipf)
    ws = bq.Workspaces("cuda")
    args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], k)
    got = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    counts = _check(sp, inp, r, got)
    if zipf > 0:
        assert counts.max() > 32, "the skewed case must have an expert with several passes"
    again = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    assert torch.equal(again.view(torch.int16), got.view(torch.int16))
    torch.cuda.synchronize()
    assert int(ws._bufs["ffn"].view(torch.int32).abs().sum()) == 0
    ws.check()


@pytest.mark.parametrize("bits", [4, 2])
def test_mid_empty_experts_and_single_rows(bits):
    """Hand-made routing: experts with 0, 1, 16, 17, 32, 33 and 70 rows."""
    sizes = {0: 1, 2: 16, 3: 17, 4: 32, 5: 33, 7: 70}            # experts 1 and 6 stay empty
    T, H, I, E, k = sum(sizes.values()), 512, 512, 8, 1
    assert bq.ffn_path(T, k, E, H, I, bits) == "mid"
    ids = np.concatenate([np.full(n, e) for e, n in sizes.items()]).astype(np.int32)
    ids = np.random.default_rng(4200 + bits).permutation(ids)[:, None]
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=4200 + bits)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    off, srt, rp, act = bq.permute(to_dev(ids), E)
    got = bq.expert_ffn(to_dev(inp.x), off, srt, act, k, wd, bits, I)
    ref = oracle.expert_ffn(inp.x, to_np(off), to_np(srt), k, inp.weights, bits, I)
    yp = bf16_np_to_f32(to_np(got))
    assert oracle.rel_fro(yp, ref) <= TOL and row_rel_err(yp, ref).max() <= TOL


@pytest.mark.parametrize("bits", [4, 2])
def test_mid_table_path_matches_arrays(bits):
    """The address-table call takes the mid path too: bit-exact with the arrays,
    every third expert read from pinned host memory."""
    T, H, I, E, k = 90, 512, 1024, 8, 2
    sp, inp, wd, r = _inputs(T, H, I, E, k, bits, 4300 + bits)
    args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], k)
    ref = bq.expert_ffn(*args, wd, bits, I)
    experts = [{n: (t[e].cpu().pin_memory() if e % 3 == 1 else t[e].clone()) for n, t in wd.items()}
               for e in range(E)]
    table = bq.expert_table(experts, bits)
    got = bq.expert_ffn_table(*args, table, bits, I)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["mid_t256_h4096_e256_k8_i1024_int4", "mid_t512_h4096_e256_k8_i1024_int4"])
def test_mid_full_size_sampled(name):
    """The configurations themselves: y_perm of the hottest, a middle and the
    coldest active expert against the oracle, every row of them."""
    sp = workload.spec(name)
    assert bq.ffn_path(sp.T, sp.k, sp.E, sp.H, sp.I, sp.bits) == "mid"
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), sp.k)
    got = bq.expert_ffn(to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], sp.k, wd, sp.bits, sp.I)
    off = to_np(r["offsets"])
    counts = np.diff(off)
    act = to_np(r["active"])
    act = act[1:1 + act[0]]
    by = sorted(act.tolist(), key=lambda e: counts[e])
    _check(sp, inp, r, got, experts=[by[-1], by[len(by) // 2], by[0]])


@pytest.mark.parametrize("bits", [4, 2])
def test_prefill_hybrid_small_experts_take_the_mid_kernel(bits):
    """On the grouped-GEMM path (T*k > 24 E) INT4 and 2-bit g128 experts with
    at most 64 rows run the mid kernel and the others the GEMMs, in one call:
    every row of both kinds against the oracle, twice on one workspace
    (bit-identical, workspace left zero)."""
    T, H, I, E, k = 400, 512, 256, 16, 4
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=4400 + bits, zipf_s=1.1)
    assert bq.ffn_path(T, k, E, H, I, bits) == "gemm"
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    bias = to_dev(inp.logit_bias) if inp.logit_bias is not None else None
    r = bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), k, bias)
    ws = bq.Workspaces("cuda")
    args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], k)
    got = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    counts = _check(sp, inp, r, got)
    act = counts[counts > 0]
    assert (act <= 64).any() and (act > 64).any(), counts
    again = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    assert torch.equal(again.view(torch.int16), got.view(torch.int16))
    torch.cuda.synchronize()
    assert int(ws._bufs["ffn"].view(torch.int32).abs().sum()) == 0
