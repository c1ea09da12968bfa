"""The seeded input generator: determinism, shapes and the stated sampling laws."""
import numpy as np
import pytest

import oracle
import workload


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, -2.5, 0.0, 1e-3], np.float32)
    b = workload.bf16_bits(vals)
    back = oracle.bf16_to_f32(b)
    assert back[0] == 1.0
    assert back[1] == 1.0                       # exactly halfway -> even (1.0)
    assert back[2] == 1.0 + 2**-7               # above halfway -> up
    assert back[3] == -2.5 and back[4] == 0.0
    assert abs(back[5] - 1e-3) <= 1e-3 * 2**-8


@pytest.mark.parametrize("name", workload.list_workloads())
def test_shapes_and_determinism(name):
    sp = workload.spec(name)
    # shrink E for the big configs so this stays a quick CPU test
    small = workload.spec(name, E=4, T=min(sp.T, 16)) if sp.E > 8 else sp
    a = workload.make_layer_inputs(small)
    b = workload.make_layer_inputs(small)
    nw = small.words_per_row
    assert a.x.shape == (small.T, small.H) and a.x.dtype == np.uint16
    assert a.w_router.shape == (small.E, small.H)
    w = a.weights
    assert w["w13_codes"].shape == (small.E, 2 * small.I, nw(small.H))
    assert w["w13_scales"].shape == (small.E, 2 * small.I, small.H // small.group)
    if small.nvfp4:
        assert w["w13_scales"].dtype == np.uint8 and w["w13_gscale"].shape == (small.E,)
    assert w["w2_codes"].shape == (small.E, small.H, nw(small.I))
    assert w["w2_scales"].shape == (small.E, small.H, small.I // small.group)
    if small.bits == 2:
        assert set(np.unique(w["w13_zeros"]).tolist()) <= {1, 2}
    for key in w:
        assert np.array_equal(w[key], b.weights[key])
    assert np.array_equal(a.x, b.x)
    c = workload.make_layer_inputs(small, set_idx=1)
    assert not np.array_equal(c.weights["w13_codes"], a.weights["w13_codes"])


def test_codes_are_uniform():
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4")
    w = workload.make_weight_set(sp)["w13_codes"]
    q = oracle.unpack_codes(w, 4)
    hist = np.bincount((q.ravel() + 8).astype(np.int64), minlength=16)
    assert hist.min() > 0.9 * hist.mean() and hist.max() < 1.1 * hist.mean()


def test_int8_codes_uniform_over_the_symmetric_range():
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", bits=8, group=32)
    w = workload.make_weight_set(sp)
    q = oracle.unpack_codes(w["w13_codes"], 8).astype(np.int64)
    assert q.min() == -127 and q.max() == 127
    hist = np.bincount((q.ravel() + 127), minlength=255)
    assert hist.min() > 0.6 * hist.mean() and hist.max() < 1.4 * hist.mean()
    assert w["w13_scales"].shape == (8, 256, 256 // 32)


def test_verify_streams_share_about_half_their_experts():
    """AR(1) activations: consecutive tokens of a stream overlap in ~50% of their top-8."""
    sp = workload.spec("verify_t16_h4096_e256_k8_i1024_int4")
    x = workload.make_x(sp)
    w_r, _ = workload.make_router(sp)
    ids, _ = oracle.topk_softmax(oracle.router_logits(x, w_r), 8)
    ov = [len(set(ids[s * 4 + j]) & set(ids[s * 4 + j + 1])) / 8 for s in range(4) for j in range(3)]
    assert 0.3 <= np.mean(ov) <= 0.7


def test_zipf_prior_skews_routing():
    sp = workload.spec("prefill_t4096_h4096_e256_k8_i1024_int4", T=256)
    w_r, bias = workload.make_router(sp)
    assert bias[0] == 0.0 and np.all(np.diff(bias) < 0)
    x = workload.make_x(sp)
    ids, _ = oracle.topk_softmax(oracle.router_logits(x, w_r, bias), 8)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts[:8].sum() > 0.25 * counts.sum()          # heavy head
    assert (counts == 0).sum() > 50                         # many cold experts at T=256
