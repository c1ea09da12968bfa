"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bars: routing ids, router logits, permutation arrays and unpacked codes
bit-exact; gates within 1e-6; bf16 outputs within 2e-2 relative Frobenius error
of the float32 oracle (tensor-wide and per row).  Full-size workloads are
checked on sampled tokens / experts that the oracle computes one by one.
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


# ------------------------------------------------------------------ unpack / dequant
@pytest.mark.parametrize("bits", [4, 2])
def test_unpack_codes_exhaustive_and_random(bits):
    P = 32 // bits
    vals = 1 << bits
    # every field value in every field position, other fields cycling
    words = []
    for pos in range(P):
        for v in range(vals):
            w = 0
            for f in range(P):
                w |= (((v + f * 3) % vals) if f != pos else v) << (bits * f)
            words.append(w)
    rng = np.random.default_rng(1)
    words = np.concatenate([np.array(words, np.uint32), rng.integers(0, 2**32, 1 << 20, dtype=np.uint32)])
    got = to_np(bq.unpack_codes(to_dev(words), bits))
    exp = oracle.unpack_codes(words, bits).ravel()
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("bits", [4, 2])
def test_dequant_bf16_is_rounded_oracle(bits):
    rng = np.random.default_rng(2)
    N, K = 96, 1024
    words = rng.integers(0, 2**32, (N, K * bits // 32), dtype=np.uint32)
    scales = workload.bf16_bits(np.abs(rng.standard_normal((N, K // 128))).astype(np.float32) * 0.03)
    zeros = rng.integers(1, 3, (N, K // 128), dtype=np.uint8) if bits == 2 else None
    got = to_np(bq.dequant_bf16(to_dev(words), to_dev(scales), to_dev(zeros), bits, N, K))
    exp = workload.bf16_bits(oracle.dequantize(words, scales, zeros, bits))
    assert np.array_equal(got, exp)


# ------------------------------------------------------------------ routing
def _check_route(x, w_r, bias, k, tokens=None):
    xd, wd = to_dev(x), to_dev(w_r)
    bd = to_dev(bias) if bias is not None else None
    ids, gates, logits = bq.route(xd, wd, k, bd, want_logits=True)
    ids, gates, logits = to_np(ids), to_np(gates), to_np(logits)
    sel = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    ref_l = oracle.router_logits(x[sel], w_r, bias)
    assert np.array_equal(logits[sel].view(np.uint32), ref_l.view(np.uint32)), "router logits differ"
    ref_ids, ref_g = oracle.topk_softmax(ref_l, k)
    assert np.array_equal(ids[sel], ref_ids)
    assert np.max(np.abs(gates[sel] - ref_g)) <= 1e-6
    return ids, gates


def test_route_tiny_and_variants():
    inp = workload.make_layer_inputs("tiny_t4_h256_e8_k2_i128_int4")
    _check_route(inp.x, inp.w_router, None, 2)
    _check_route(inp.x, inp.w_router, None, 8)                                  # k = E
    bias = np.linspace(0.3, -0.3, 8).astype(np.float32)
    _check_route(inp.x, inp.w_router, bias, 3)
    w = inp.w_router.copy()
    w[5] = w[2]
    w[6] = w[2]                                                                 # exact ties
    ids, _ = _check_route(inp.x, w, None, 8)
    for t in range(ids.shape[0]):
        pos = {int(e): i for i, e in enumerate(ids[t])}
        assert pos[2] < pos[5] < pos[6]


@pytest.mark.parametrize("T,H,E,k", [(33, 512, 300, 8), (100, 256, 64, 6), (17, 1024, 1024, 32), (32, 384, 7, 7),
                                     (5, 2048, 13, 4), (1, 4096, 6, 2)])
def test_route_both_kernels_ragged_shapes(T, H, E, k):
    """The small router with the rows staged in LDS (H a power of two from 512
    to 4096; ragged expert groups and token pairs) and with slice-per-lane
    loads (other H)."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, E=E, k=k, seed=77 + T)
    x = workload.make_x(sp)
    w_r, _ = workload.make_router(sp)
    bias = (np.random.default_rng(T).standard_normal(E) * 0.01).astype(np.float32)
    _check_route(x, w_r, bias, k)


@pytest.mark.parametrize("T,H,E,k", [(33, 2048, 300, 8), (1024, 2048, 64, 4), (1025, 2048, 64, 4), (100, 4096, 1, 1),
                                     (257, 2048, 1024, 32), (40, 4096, 256, 8)])
def test_route_tiles_kernel_ragged_shapes(T, H, E, k):
    """32 < T <= 1024 with H % 2048 == 0 runs the logits as tiles of tokens x
    64 experts x 4 K parts and the top-k (with the tree's top levels) as a
    second launch: ragged token tiles and expert groups against the oracle,
    the logits written to the caller's array; then the same call without
    logits gives the same ids and gates and leaves the workspace zero.
    T = 1025 checks the token-tiled kernel across the boundary."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, E=E, k=k, seed=88 + T)
    x = workload.make_x(sp)
    w_r, _ = workload.make_router(sp)
    bias = (np.random.default_rng(T).standard_normal(E) * 0.01).astype(np.float32)
    ids, gates = _check_route(x, w_r, bias, k)
    ws = bq.Workspaces("cuda")
    for _ in range(2):
        ids2, gates2 = bq.route(to_dev(x), to_dev(w_r), k, to_dev(bias), ws=ws)
        assert np.array_equal(to_np(ids2), ids) and np.array_equal(to_np(gates2), gates)
        torch.cuda.synchronize()
        assert int(ws._bufs["route"].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("name", ["decode_t1_h4096_e256_k8_i1024_int4", "verify_t16_h4096_e256_k8_i1024_int4"])
def test_route_decode_full_size(name):
    sp = workload.spec(name)
    w_r, bias = workload.make_router(sp)
    for s in range(3):
        _check_route(workload.make_x(sp, s), w_r, bias, sp.k)


@pytest.mark.parametrize("name", ["prefill_t4096_h4096_e256_k8_i1024_int4", "prefill_t8192_h4096_e256_k8_i1024_int2"])
def test_route_prefill_full_size_all_tokens(name):
    """The token-tiled prefill router against the oracle on every token: logit
    bits, ids and gates (near-ties under the Zipf prior included)."""
    sp = workload.spec(name)
    w_r, bias = workload.make_router(sp)
    x = workload.make_x(sp)
    ids, _ = _check_route(x, w_r, bias, sp.k)
    say(f"    {sp.T} tokens: logits, ids and gates match the oracle")


# ------------------------------------------------------------------ permutation
def test_permute_workspace_reused_and_left_zero():
    """Batches above 4096 rows keep per-block counts in the workspace: three
    calls of different sizes on one workspace each equal the oracle, and the
    workspace is zero after each."""
    ws = bq.Workspaces("cuda")
    for i, (T, E) in enumerate([(8192, 256), (600, 256), (5000, 256), (8192, 256)]):
        rng = np.random.default_rng(900 + i)
        ids = rng.integers(0, E, (T, 8)).astype(np.int32)
        off, sr, rp, act = [to_np(v) for v in bq.permute(to_dev(ids), E, ws=ws)]
        r_off, r_sr, r_rp, r_act = oracle.permute(ids, E)
        assert np.array_equal(off, r_off) and np.array_equal(sr, r_sr) and np.array_equal(rp, r_rp), (T, E)
        assert np.array_equal(act, r_act), (T, E)
        torch.cuda.synchronize()
        if "permute" in ws._bufs:
            assert int(ws._bufs["permute"].view(torch.int32).abs().sum()) == 0, (T, E)



@pytest.mark.parametrize("T,k,E,bad", [(1, 8, 256, False), (16, 8, 256, False), (4, 2, 8, True), (4096, 8, 256, False),
                                       (8192, 8, 256, True), (700, 3, 1024, True), (5, 1, 1, False), (300, 32, 40, False),
                                       (4097, 1, 1024, True), (1025, 4, 1, False), (512, 8, 256, False),
                                       (513, 8, 256, True), (60000, 8, 384, True)])
def test_permute_bit_exact(T, k, E, bad):
    rng = np.random.default_rng(T * 7 + E)
    ids = np.stack([rng.permutation(E)[:k] if k <= E else rng.integers(0, E, k) for _ in range(T)]).astype(np.int32)
    if T > 64:  # skewed: many rows on a few experts
        hot = rng.random((T, k)) < 0.5
        ids[hot] = rng.integers(0, max(1, E // 16), hot.sum())
    if bad:
        m = rng.random((T, k)) < 0.05
        ids[m] = rng.choice([-1, E, E + 5], m.sum())
    off, sr, rp, act = [to_np(v) for v in bq.permute(to_dev(ids), E)]
    valid = (ids >= 0) & (ids < E)
    flat = ids.ravel()
    vflat = np.where(valid.ravel(), flat, E)          # invalid rows sort after every expert
    r_off, r_sr, r_rp, r_act = oracle.permute(np.minimum(vflat, E).reshape(T, k), E + 1)
    nvalid = int(valid.sum())
    assert np.array_equal(off, r_off[:E + 1]), "offsets"
    assert off[E] == nvalid
    assert np.array_equal(sr[:nvalid], r_sr[:nvalid]), "sorted_rows"
    exp_rp = np.where(valid.ravel(), r_rp, -1)
    assert np.array_equal(rp, exp_rp), "row_pos"
    exp_act = [e for e in range(E) if (flat == e).any()]
    assert act[0] == len(exp_act)
    assert act[1:1 + len(exp_act)].tolist() == exp_act
    assert np.all(act[1 + len(exp_act):] == -1)


@pytest.mark.parametrize("T,H,E,k", [(1, 4096, 256, 8), (16, 4096, 256, 8), (32, 512, 256, 8), (33, 256, 64, 8),
                                     (3, 256, 1024, 32), (32, 384, 7, 7), (5, 256, 1, 1), (8, 256, 300, 32),
                                     (2, 4096, 8, 2), (9, 1024, 100, 29)])
def test_route_permute_matches_route_then_permute(T, H, E, k):
    """The one-launch router + grouping gives the outputs of moe_route and moe_permute bit for bit."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, E=E, k=k, seed=300 + T + E)
    w_r, _ = workload.make_router(sp)
    bias = (np.random.default_rng(E).standard_normal(E) * 0.01).astype(np.float32)
    ws = bq.Workspaces("cuda:0")
    wd, bd = to_dev(w_r), to_dev(bias)
    for s in range(3):                                  # reused workspace: the control block is left zeroed
        x = workload.make_x(sp, s)
        got = {n: to_np(v) for n, v in bq.route_permute(to_dev(x), wd, k, bd, want_logits=True, ws=ws).items()}
        ref_l = oracle.router_logits(x, w_r, bias)
        assert np.array_equal(got["logits"].view(np.uint32), ref_l.view(np.uint32)), "router logits differ"
        ref_ids, ref_g = oracle.topk_softmax(ref_l, k)
        assert np.array_equal(got["ids"], ref_ids)
        assert np.max(np.abs(got["gates"] - ref_g)) <= 1e-6
        r_off, r_sr, r_rp, r_act = oracle.permute(ref_ids, E)
        assert np.array_equal(got["offsets"], r_off), "offsets"
        assert np.array_equal(got["sorted_rows"], r_sr), "sorted_rows"
        assert np.array_equal(got["row_pos"], r_rp), "row_pos"
        assert np.array_equal(got["active"][:1 + got["active"][0]], r_act[:1 + r_act[0]]), "active"
        assert np.all(got["active"][1 + got["active"][0]:] == -1)
        sep_ids, sep_g = bq.route(to_dev(x), wd, k, bd, ws=ws)
        sep = [to_np(v) for v in bq.permute(sep_ids, E, ws=ws)]
        assert np.array_equal(to_np(sep_ids), got["ids"]) and np.array_equal(to_np(sep_g), got["gates"])
        for a, b in zip(sep, [got["offsets"], got["sorted_rows"], got["row_pos"], got["active"]]):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("T,k,H", [(37, 8, 4096), (5, 12, 1000)])
def test_combine_matches_oracle(T, k, H):
    """k = 12 reads the rows in a batch of 8 and a ragged one of 4; H = 1000
    leaves the last block's threads partly past H; invalid row positions (a
    dropped row, one past the end) add nothing."""
    rng = np.random.default_rng(3 + k)
    y_perm = workload.bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32))
    row_pos = rng.permutation(T * k).astype(np.int32)
    row_pos[5] = -1
    row_pos[min(9, T * k - 1)] = T * k + 3
    g = rng.random((T, k)).astype(np.float32)
    got = bf16_np_to_f32(to_np(bq.combine(to_dev(y_perm), to_dev(row_pos), to_dev(g))))
    yp = bf16_np_to_f32(y_perm)
    rp = row_pos.copy()
    yp_ext = np.concatenate([yp, np.zeros((1, H), np.float32)])
    rp[(rp < 0) | (rp >= T * k)] = T * k
    ref = oracle.combine(yp_ext, rp, g)
    assert oracle.rel_fro(got, ref) < 4e-3
    assert np.max(row_rel_err(got, ref)) < 8e-3


# ------------------------------------------------------------------ whole layer
def _layer(inp, weights_dev=None, k=None):
    sp = inp.spec
    wd = weights_dev or weights_to_dev(inp.weights)
    out = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), to_dev(inp.logit_bias) if inp.logit_bias is not None else None,
                       wd, k or sp.k, sp.bits, sp.I, want_logits=True)
    return {kk: to_np(v) for kk, v in out.items()}, wd


def _check_layer_exact(inp, got, k=None):
    sp = inp.spec
    ref = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, k or sp.k, sp.bits, sp.I)
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32))
    for key in ("ids", "offsets", "sorted_rows", "row_pos", "active"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.max(np.abs(got["gates"] - ref["gates"])) <= 1e-6
    yp = bf16_np_to_f32(got["y_perm"])
    y = bf16_np_to_f32(got["y"])
    e1, e2 = oracle.rel_fro(yp, ref["y_perm"]), oracle.rel_fro(y, ref["y"])
    say(f"    y_perm rel-fro {e1:.2e}, y rel-fro {e2:.2e}")
    assert e1 <= TOL and e2 <= TOL
    assert np.max(row_rel_err(yp, ref["y_perm"])) <= TOL
    if max(e1, e2) > 5e-3:
        say(f"    ALARM: error above the expected ~3e-3 ({e1:.2e}, {e2:.2e})")
    return ref


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("T", [1, 4, 16, 17, 40, 300])
def test_layer_small_shapes_both_paths(bits, T):
    """T <= 16 runs the decode GEMV, T > 16 the grouped MFMA GEMM (ragged tiles)."""
    kw = dict(T=T)
    if bits == 2:
        kw.update(bits=2, scale_sigma=0.05)
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", seed=500 + T + bits, **kw)
    inp = workload.make_layer_inputs(sp)
    got, _ = _layer(inp)
    _check_layer_exact(inp, got)


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_mid_shapes(bits):
    """H = 1024, I = 256, E = 32, top-4: several K tiles, both paths, several N blocks."""
    for T in (3, 16, 200):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=1024, I=256, E=32, k=4, bits=bits,
                           scale_sigma=0.02 if bits == 4 else 0.05, seed=900 + T)
        inp = workload.make_layer_inputs(sp)
        got, _ = _layer(inp)
        _check_layer_exact(inp, got)


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_decode_shapes_of_the_full_model(bits):
    """H = 4096, I = 1024 (the decode kernel's full-chunk path) with few experts:
    T = 1, a few tokens with experts holding 1-2 rows, and T = 16 with E = 8
    (experts holding more rows than one pass stages)."""
    for T, E, k in ((1, 8, 2), (3, 8, 2), (16, 8, 4)):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=4096, I=1024, E=E, k=k, bits=bits,
                           scale_sigma=0.02 if bits == 4 else 0.05, seed=1200 + T)
        inp = workload.make_layer_inputs(sp)
        got, _ = _layer(inp)
        _check_layer_exact(inp, got)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_layer_deterministic_and_workspace_left_zero(T):
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=512, I=256, E=16, k=4)
    inp = workload.make_layer_inputs(sp)
    ws = bq.Workspaces("cuda")
    wd = weights_to_dev(inp.weights)
    args = (to_dev(inp.x), to_dev(inp.w_router), None, wd, sp.k, sp.bits, sp.I)
    a = bq.moe_layer(*args, ws=ws)
    b = bq.moe_layer(*args, ws=ws)
    for key in a:
        ta, tb = a[key], b[key]
        if ta.dtype == torch.bfloat16:
            ta, tb = ta.view(torch.int16), tb.view(torch.int16)
        assert torch.equal(ta, tb), key
    torch.cuda.synchronize()
    for name, buf in ws._bufs.items():
        assert int(buf.view(torch.int32).abs().sum()) == 0, name  # every workspace is all-zero between calls


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("shape", ["tiny", "mid", "full"])
def test_layer_fused_matches_stages(bits, shape):
    """moe_layer_* (one launch) gives the stage calls' y, ids and gates bit for bit, and the oracle's y."""
    dims = dict(tiny=dict(H=256, I=128, E=8, k=2), mid=dict(H=1024, I=256, E=32, k=4),
                full=dict(H=4096, I=1024, E=256, k=8))[shape]
    ws = bq.Workspaces("cuda")
    Ts = (1, 2, 5, 8, 16) if shape != "full" else (1, 8, 16)
    for T in Ts:
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, bits=bits, scale_sigma=0.02 if bits == 4 else 0.05,
                           seed=2000 + T + bits, **dims)
        inp = workload.make_layer_inputs(sp)
        wd = weights_to_dev(inp.weights)
        bias = to_dev(inp.logit_bias) if inp.logit_bias is not None else None
        for rep in range(2):                                        # the workspace is reused
            y, ids, gates = bq.layer(to_dev(inp.x), to_dev(inp.w_router), bias, wd, sp.k, sp.bits, sp.I, ws=ws,
                                     want_routing=True)
            st = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), bias, wd, sp.k, sp.bits, sp.I, ws=ws)
            assert torch.equal(ids, st["ids"]), (T, rep)
            assert torch.equal(gates.view(torch.int32), st["gates"].view(torch.int32)), (T, rep)
            assert torch.equal(y.view(torch.int16), st["y"].view(torch.int16)), (T, rep)
        say(f"    fused layer T={T}: bit-exact with the stages")
        if shape != "full" or T == 1:                               # the stages are checked at full size elsewhere
            ref = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, sp.bits, sp.I)
            assert oracle.rel_fro(bf16_np_to_f32(to_np(y)), ref["y"]) <= TOL
    torch.cuda.synchronize()
    for name, buf in ws._bufs.items():
        assert int(buf.view(torch.int32).abs().sum()) == 0, name


def test_layer_fused_rejects_large_batches():
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=17)
    inp = workload.make_layer_inputs(sp)
    with pytest.raises(bq.MoEError, match="stages"):
        bq.layer(to_dev(inp.x), to_dev(inp.w_router), None, weights_to_dev(inp.weights), sp.k, sp.bits, sp.I)


@pytest.mark.parametrize("bits", [4, 2])
def test_layer_one_workspace_across_paths(bits):
    """Decode and grouped-GEMM calls alternate on one set of workspaces: no call sees another's h."""
    ws = bq.Workspaces("cuda")
    for i, T in enumerate([1, 40, 1, 16, 300, 3, 1, 17, 2]):
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=512, I=256, E=16, k=4, bits=bits,
                           scale_sigma=0.02 if bits == 4 else 0.05, seed=1300 + 10 * i + bits)
        inp = workload.make_layer_inputs(sp)
        out = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), None, weights_to_dev(inp.weights), sp.k, sp.bits,
                           sp.I, ws=ws, want_logits=True)
        _check_layer_exact(inp, {kk: to_np(v) for kk, v in out.items()})
    torch.cuda.synchronize()
    assert int(ws._bufs["ffn"].view(torch.int32).abs().sum()) == 0


def test_layer_all_experts_one_token_each_and_empty_experts():
    # k = E: every expert active; T = 2 with E = 8 and k = 1: empty experts
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=3, k=8)
    inp = workload.make_layer_inputs(sp)
    got, _ = _layer(inp)
    _check_layer_exact(inp, got)
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=2, k=1)
    inp = workload.make_layer_inputs(sp)
    got, _ = _layer(inp)
    _check_layer_exact(inp, got)


# ------------------------------------------------------------------ full-size workloads
def _full_decode(name, n_sets=2):
    sp = workload.spec(name)
    w_r, bias = workload.make_router(sp)
    ws = bq.Workspaces("cuda")
    for s in range(n_sets):
        inp = workload.LayerInputs(sp, workload.make_x(sp, s), w_r, bias, workload.make_weight_set(sp, s))
        wd = weights_to_dev(inp.weights)
        out = bq.moe_layer(to_dev(inp.x), to_dev(w_r), to_dev(bias) if bias is not None else None, wd, sp.k,
                           sp.bits, sp.I, ws=ws, want_logits=True)
        got = {kk: to_np(v) for kk, v in out.items()}
        _check_layer_exact(inp, got)
        del wd, out
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["decode_t1_h4096_e256_k8_i1024_int4", "decode_t1_h4096_e256_k8_i1024_int2",
                                  "verify_t16_h4096_e256_k8_i1024_int4"])
def test_layer_decode_full_size(name):
    _full_decode(name, n_sets=2 if "t1_" in name else 1)


@pytest.mark.parametrize("bits", [4, 2])
def test_decode_ffn_item_queues_repeatable(bits):
    """More decode items than co-resident blocks (H = 4096, I = 1024, 32
    experts, T = 16, top-4: about 3000 items over 768 blocks), so blocks past
    their first item draw from the per-XCD item queues: y_perm against the
    oracle on every row, a second call on the same workspace bit-identical,
    and the workspace (queue counters included) left zero."""
    T, H, I, E, k = 16, 4096, 1024, 32, 4
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, bits=bits,
                       scale_sigma=0.02 if bits == 4 else 0.05, seed=5100 + bits)
    assert bq.ffn_path(T, k, E, H, I, bits) == "decode"
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    r = bq.route_permute(to_dev(inp.x), to_dev(inp.w_router), k)
    act = to_np(r["active"])
    assert int(act[0]) * (I // 16 + H // 128) > 768, "the case must have more items than one round of blocks"
    ws = bq.Workspaces("cuda")
    args = (to_dev(inp.x), r["offsets"], r["sorted_rows"], r["active"], k)
    got = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    again = bq.expert_ffn(*args, wd, bits, I, ws=ws)
    assert torch.equal(again.view(torch.int16), got.view(torch.int16))
    torch.cuda.synchronize()
    assert int(ws._bufs["ffn"].view(torch.int32).abs().sum()) == 0
    ws.check()
    off, srt = to_np(r["offsets"]), to_np(r["sorted_rows"])
    ref = oracle.expert_ffn(inp.x, off, srt, k, inp.weights, bits, I)
    yp = bf16_np_to_f32(to_np(got))
    assert oracle.rel_fro(yp, ref) <= TOL and row_rel_err(yp, ref).max() <= TOL


@pytest.mark.parametrize("name", ["prefill_t4096_h4096_e256_k8_i1024_int4", "prefill_t8192_h4096_e256_k8_i1024_int2",
                                  "mid_t64_h4096_e256_k8_i1024_int4"])
def test_layer_prefill_full_size_sampled(name):
    """Routing and permutation of every token against the oracle's own (logit
    bits, ids, gates; offsets, sorted_rows, row_pos, active from the oracle's
    ids); the FFN output on sampled experts and tokens the oracle computes one
    by one."""
    sp = workload.spec(name)
    inp = workload.make_layer_inputs(sp)
    wd = weights_to_dev(inp.weights)
    out = bq.moe_layer(to_dev(inp.x), to_dev(inp.w_router), to_dev(inp.logit_bias) if inp.logit_bias is not None
                       else None, wd, sp.k, sp.bits, sp.I, want_logits=True)
    got = {kk: to_np(v) for kk, v in out.items()}
    ref_l = oracle.router_logits(inp.x, inp.w_router, inp.logit_bias)
    assert np.array_equal(got["logits"].view(np.uint32), ref_l.view(np.uint32)), "router logits differ"
    ref_ids, ref_g = oracle.topk_softmax(ref_l, sp.k)
    assert np.array_equal(got["ids"], ref_ids), "ids"
    assert np.max(np.abs(got["gates"] - ref_g)) <= 1e-6
    r_off, r_sr, r_rp, r_act = oracle.permute(ref_ids, sp.E)
    for key, r in (("offsets", r_off), ("sorted_rows", r_sr), ("row_pos", r_rp), ("active", r_act)):
        assert np.array_equal(got[key], r), key
    say(f"    routing and permutation of all {sp.T} tokens bit-exact")
    counts = np.diff(got["offsets"])
    say(f"    rows/expert: max {counts.max()}, empty {(counts == 0).sum()}, <81: {(counts < 81).sum()}")
    # sampled experts: the hottest, a middle one, the coldest non-empty one
    act = got["active"][1:1 + got["active"][0]]
    by = sorted(act.tolist(), key=lambda e: counts[e])
    experts = [by[-1], by[len(by) // 2], by[0]]
    yp_ref = oracle.expert_ffn(inp.x, got["offsets"], got["sorted_rows"], sp.k, inp.weights, sp.bits, sp.I,
                               experts=experts)
    yp = bf16_np_to_f32(got["y_perm"])
    for e in experts:
        o0, o1 = got["offsets"][e], got["offsets"][e + 1]
        err = oracle.rel_fro(yp[o0:o1], yp_ref[o0:o1])
        say(f"    expert {e} ({o1 - o0} rows): y_perm rel-fro {err:.2e}")
        assert err <= TOL
        assert np.max(row_rel_err(yp[o0:o1], yp_ref[o0:o1])) <= TOL
    # sampled tokens end to end (routing, gates and output)
    tok = np.concatenate([np.random.default_rng(9).choice(sp.T, 6, replace=False), [0, sp.T - 1]])
    ref = oracle.moe_layer_tokens(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, sp.bits, sp.I, tok)
    assert np.array_equal(got["ids"][tok], ref["ids"])
    assert np.max(np.abs(got["gates"][tok] - ref["gates"])) <= 1e-6
    y = bf16_np_to_f32(got["y"][tok])
    err = oracle.rel_fro(y, ref["y"])
    say(f"    sampled tokens y rel-fro {err:.2e}")
    assert err <= TOL
