"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names the step (O1..O8 in oracle/moe_oracle.py) it pins and the kind
of pin: a hand-derived golden value (tests/golden), a closed form, brute force
on tiny inputs, or an invariant.  They are chosen so that a plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, a wrong
summation order, a wrong tie rule) fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals):
    return workload.bf16_bits(np.asarray(vals, dtype=np.float32))


# ------------------------------------------------------------------ O5 unpack
def _golden_unpack():
    rows = []
    for line in open(os.path.join(GOLDEN, "unpack_codes.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        rows.append((int(parts[0]), int(parts[1], 16), [int(v) for v in parts[2:]]))
    return rows


def test_unpack_matches_hand_derived_golden():
    rows = _golden_unpack()
    assert len(rows) >= 12
    for bits, word, codes in rows:
        got = oracle.unpack_codes(np.array([word], dtype=np.uint32), bits)
        assert got.tolist() == codes, (bits, hex(word))


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_pack_unpack_exhaustive_every_code_every_field(bits):
    """Every code value in every field position of a word round-trips."""
    P = 32 // bits
    lo, hi = {4: (-8, 7), 2: (0, 3), 8: (-127, 127)}[bits]
    codes = np.arange(lo, hi + 1)
    rows = []
    for pos in range(P):
        for c in codes:
            filler = lo if c != lo else hi
            r = np.full(P, filler, dtype=np.int16)
            r[pos] = c
            rows.append(r)
    q = np.stack(rows)
    w = oracle.pack_codes(q, bits)
    back = oracle.unpack_codes(w, bits)
    assert np.array_equal(back, q)
    # field position: the code at position pos lives in bits [b*pos, b*pos+b)
    for r, word in zip(rows, w[:, 0].tolist()):
        for pos in range(P):
            field = (word >> (bits * pos)) & ((1 << bits) - 1)
            assert field == (int(r[pos]) + {4: 8, 2: 0, 8: 128}[bits])


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_unpack_pack_random_words_roundtrip(bits):
    rng = np.random.default_rng(7)
    w = rng.integers(0, 2**32, size=(5, 9), dtype=np.uint32)
    assert np.array_equal(oracle.pack_codes(oracle.unpack_codes(w, bits), bits), w)


def test_unpack_k_order_across_words():
    """Code of K index k lives in word k // P (K-packing, not N-packing)."""
    q = np.arange(32, dtype=np.int16) % 16 - 8          # K = 32 distinct-ish codes
    w = oracle.pack_codes(q[None, :], 4)
    assert w.shape == (1, 4)
    assert w[0, 0] == 0x76543210 and w[0, 1] == 0xFEDCBA98


# ------------------------------------------------------------------ O6 dequant
def test_dequant_golden_values():
    # INT4: word 0xFEDCBA98 holds q = 0..7; scale 0.5 -> 0, 0.5, ..., 3.5
    words = np.full((1, 16), 0xFEDCBA98, dtype=np.uint32)          # K = 128
    s = _bf16([[0.5]])
    W = oracle.dequantize(words, s, None, 4)
    assert W[0, :8].tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 3.5]
    # 2-bit: word 0xE4E4E4E4 holds u = 0,1,2,3,...; zero-point 2, scale 2.0 -> -4,-2,0,2
    words2 = np.full((1, 8), 0xE4E4E4E4, dtype=np.uint32)          # K = 128
    W2 = oracle.dequantize(words2, _bf16([[2.0]]), np.array([[2]], np.uint8), 2)
    assert W2[0, :4].tolist() == [-4.0, -2.0, 0.0, 2.0]


@pytest.mark.parametrize("bits", [4, 2, 8])
def test_dequant_unit_scale_zero_point_gives_codes(bits):
    rng = np.random.default_rng(3)
    N, K = 3, 256
    w = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint32)
    ones = _bf16(np.ones((N, K // 128)))
    z = np.zeros((N, K // 128), np.uint8) if bits == 2 else None
    W = oracle.dequantize(w, ones, z, bits)
    assert np.array_equal(W, oracle.unpack_codes(w, bits).astype(np.float32))


@pytest.mark.parametrize("bits", [4, 2])
def test_dequant_group_boundaries(bits):
    """Scale/zero of group g affects exactly columns [128g, 128g+128) of its row."""
    rng = np.random.default_rng(11)
    N, K = 4, 512
    w = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint32)
    s = _bf16(np.abs(rng.standard_normal((N, K // 128))) + 0.1)
    z = rng.integers(1, 3, size=(N, K // 128), dtype=np.uint8) if bits == 2 else None
    base = oracle.dequantize(w, s, z, bits)
    for n, g in [(0, 0), (2, 3), (3, 1)]:
        s2 = s.copy()
        s2[n, g] = _bf16([[8.0]])[0, 0]
        z2 = None if z is None else z.copy()
        if z2 is not None:
            z2[n, g] = 0
        moved = oracle.dequantize(w, s2, z2, bits)
        diff = np.argwhere(moved != base)
        assert diff.size > 0
        assert set(diff[:, 0].tolist()) == {n}
        assert diff[:, 1].min() >= 128 * g and diff[:, 1].max() < 128 * (g + 1)


def test_dequant_golden_values_group32_and_int8():
    # INT8 word 0x81818181 holds q = 1 in every byte; K = 128 in four groups of
    # 32 with scales 0.5, 1, 2, 4 -> 32 copies of each scale, in K order
    words = np.full((1, 32), 0x81818181, dtype=np.uint32)
    W = oracle.dequantize(words, _bf16([[0.5, 1.0, 2.0, 4.0]]), None, 8, group=32)
    assert W[0].tolist() == [0.5] * 32 + [1.0] * 32 + [2.0] * 32 + [4.0] * 32
    # INT4 word 0x0F0F0F0F holds q = 7, -8, 7, -8, ...; group 32, scales 1 and -0.25
    w4 = np.full((1, 8), 0x0F0F0F0F, dtype=np.uint32)               # K = 64
    W4 = oracle.dequantize(w4, _bf16([[1.0, -0.25]]), None, 4, group=32)
    assert W4[0, :4].tolist() == [7.0, -8.0, 7.0, -8.0]
    assert W4[0, 32:36].tolist() == [-1.75, 2.0, -1.75, 2.0]
    # INT8 extremes: 0x01 -> -127, 0xFF -> 127
    W8 = oracle.dequantize(np.full((1, 32), 0xFF01FF01, dtype=np.uint32), _bf16([[0.5]]), None, 8)
    assert W8[0, :4].tolist() == [-63.5, 63.5, -63.5, 63.5]


@pytest.mark.parametrize("bits", [4, 8])
def test_dequant_group32_boundaries_and_reduction_to_group128(bits):
    """With group 32, scale j of a row moves exactly columns [32j, 32j+32); four
    equal scales per 128 columns give the group-128 result."""
    rng = np.random.default_rng(21)
    N, K = 3, 256
    w = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint32)
    s = _bf16(np.abs(rng.standard_normal((N, K // 32))) + 0.1)
    base = oracle.dequantize(w, s, None, bits, group=32)
    for n, j in [(0, 0), (1, 5), (2, 7)]:
        s2 = s.copy()
        s2[n, j] = _bf16([[8.0]])[0, 0]
        diff = np.argwhere(oracle.dequantize(w, s2, None, bits, group=32) != base)
        assert set(diff[:, 0].tolist()) == {n}
        assert diff[:, 1].min() >= 32 * j and diff[:, 1].max() < 32 * (j + 1)
    s128 = _bf16(np.abs(rng.standard_normal((N, K // 128))) + 0.1)
    assert np.array_equal(oracle.dequantize(w, np.repeat(s128, 4, axis=1), None, bits, group=32),
                          oracle.dequantize(w, s128, None, bits, group=128))


@pytest.mark.parametrize("group", [32, 128])
def test_int8_every_code_every_group_position_scale_and_activation_extremes(group):
    """The pages' int8 battery, applied to the oracle: each code -127..127 at
    each position of a group, under extreme scales and activations, gives the
    product code * scale * x exactly (checked in exact rationals)."""
    from fractions import Fraction
    scales = [2.0 ** -14, 1.0, 2.0 ** 7]                     # bf16-exact scale extremes
    acts = [2.0 ** -10, -1.0, 2.0 ** 6]                      # bf16-exact activation extremes
    codes = np.arange(-127, 128)
    K = group
    for pos in range(0, group, 3 if group == 128 else 1):
        q = np.zeros((codes.size, K), np.int16)
        q[:, pos] = codes
        words = oracle.pack_codes(q, 8)
        for sc in scales:
            W = oracle.dequantize(words, _bf16(np.full((codes.size, 1), sc)), None, 8, group=group)
            nz = np.flatnonzero(W.any(axis=0))
            assert nz.tolist() in ([pos], [])
            for xv in acts:
                x = np.zeros(K, np.float32)
                x[pos] = xv
                y = W.astype(np.float64) @ x.astype(np.float64)
                for c, yv in zip(codes[::17], y[::17]):
                    assert Fraction(float(yv)) == Fraction(int(c)) * Fraction(sc) * Fraction(xv)


# ------------------------------------------------------------------ FP6 e2m3
def _golden_fp6():
    vals, packs = {}, []
    for line in open(os.path.join(GOLDEN, "fp6_e2m3.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "pack":
            packs.append((int(parts[1]), [int(w, 16) for w in parts[2:5]]))
        else:
            vals[int(parts[0])] = float(parts[1])
    return vals, packs


def _pack_stream(codes):
    """Test-side writer of the FP6 bit stream, one bit at a time."""
    codes = list(codes)
    words = [0] * (len(codes) * 6 // 32)
    for k, c in enumerate(codes):
        for b in range(6):
            if (c >> b) & 1:
                words[(6 * k + b) // 32] |= 1 << ((6 * k + b) % 32)
    return np.array(words, np.uint32)


def test_fp6_values_match_hand_written_table():
    vals, _ = _golden_fp6()
    assert sorted(vals) == list(range(64))
    got = oracle.e2m3_value(np.arange(64))
    for c in range(64):
        assert got[c] == vals[c] and math.copysign(1.0, got[c]) == math.copysign(1.0, vals[c]), c
    # every value is exact in bf16
    assert np.array_equal(oracle.bf16_to_f32(_bf16(got)), got)


def test_fp6_packing_hand_packed_rows():
    _, packs = _golden_fp6()
    assert len(packs) >= 3
    for c, words in packs:
        assert oracle.unpack_fp6_fields(np.array([words], np.uint32)).tolist() == [[c] * 16]
        assert _pack_stream([c] * 16).tolist() == words


def test_fp6_every_code_every_position_and_scale_extremes():
    """Each code at each position of a 128-K group, under fp16 scale extremes,
    dequantises to value * scale exactly (exact rationals) and nowhere else."""
    from fractions import Fraction
    vals, _ = _golden_fp6()
    scales = [2.0 ** -14, 1.0, 65504.0]                      # fp16 min normal, one, max
    for pos in range(0, 128, 5):
        rows = []
        for c in range(64):
            codes = [0] * 128
            codes[pos] = c
            rows.append(_pack_stream(codes))
        words = np.stack(rows)
        assert np.array_equal(oracle.unpack_fp6_fields(words)[:, pos], np.arange(64))
        for sc in scales:
            s16 = np.full((64, 1), np.float16(sc)).view(np.uint16)
            W = oracle.dequantize(words, s16, None, 6)
            others = np.delete(W, pos, axis=1)
            assert not others.any()
            for c in range(0, 64, 3):
                assert Fraction(float(W[c, pos])) == Fraction(vals[c]) * Fraction(sc)


def test_fp6_random_rows_against_bitwise_reader():
    rng = np.random.default_rng(31)
    words = rng.integers(0, 2**32, size=(3, 24), dtype=np.uint32)   # K = 128
    fields = oracle.unpack_fp6_fields(words)
    for n in range(3):
        stream = 0
        for i, w in enumerate(words[n].tolist()):
            stream |= w << (32 * i)
        assert fields[n].tolist() == [(stream >> (6 * k)) & 63 for k in range(128)]


# ------------------------------------------------------------------ NVFP4
def _golden_nvfp4():
    rows = {"e2m1": [], "e4m3": [], "r2": [], "r8": []}
    for line in open(os.path.join(GOLDEN, "nvfp4.txt")):
        line = line.split("#")[0].strip()
        if line:
            t, a, b = line.split()
            rows[t].append((int(a, 0) if t in ("e2m1", "e4m3") else float(a), float(b)))
    return rows


def test_nvfp4_codes_and_rounding_match_hand_written_values():
    g = _golden_nvfp4()
    assert len(g["e2m1"]) == 16 and len(g["e4m3"]) >= 8
    for c, v in g["e2m1"]:
        got = float(oracle.e2m1_value(np.array([c]))[0])
        assert got == v and math.copysign(1, got) == math.copysign(1, v), c
    for c, v in g["e4m3"]:
        assert float(oracle.e4m3_value(np.array([c]))[0]) == v, hex(c)
    for a, b in g["r2"]:
        assert float(oracle.round_e2m1(np.array([a]))[0]) == b, a
    for a, b in g["r8"]:
        assert float(oracle.round_e4m3(np.array([a]))[0]) == b, a


def test_nvfp4_rounding_lands_on_the_grids_and_is_nearest():
    """Brute force: every rounding result is a grid value, and no grid value is nearer."""
    rng = np.random.default_rng(41)
    grid2 = np.unique(np.abs(oracle.e2m1_value(np.arange(16))))
    grid8 = np.unique(oracle.e4m3_value(np.arange(0x7F)))
    for grid, fn, hi in ((grid2, oracle.round_e2m1, 6.0), (grid8, oracle.round_e4m3, 448.0)):
        v = np.abs(rng.standard_normal(4000)).astype(np.float32) * np.float32(hi / 3)
        r = fn(v)
        assert np.isin(r, grid).all()
        d = np.abs(v[:, None].astype(np.float64) - grid[None, :])
        best = d.min(axis=1)
        assert np.all(np.abs(v - r) <= best + 1e-12)


def test_nvfp4_quantiser_properties():
    """Group scale from the group maximum; values exact multiples of it; zero
    groups stay zero; a group already on the grid comes back as its codes times
    its scale (the tensor scale is applied after the product)."""
    rng = np.random.default_rng(43)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    x[2, 16:32] = 0.0
    G = 2.0 ** -8
    s, xq = oracle.quant_nvfp4(x, G)
    assert s.shape == (5, 4) and xq.shape == x.shape
    assert np.all(s[2, 1] == 0) and not xq[2, 16:32].any()
    grid = np.unique(np.abs(oracle.e2m1_value(np.arange(16))))
    ratio = np.abs(xq.reshape(5, 4, 16)) / np.where(s > 0, s, 1)[..., None]
    assert np.isin(ratio, grid).all()
    amax = np.abs(x.reshape(5, 4, 16)).max(-1)
    assert np.allclose(s[s > 0], (amax / (6 * G))[s > 0], rtol=2 ** -4)
    # a group already on the grid with scale exactly amax / (6 G) quantises to itself
    y = np.zeros((1, 16), np.float32)
    y[0, :8] = np.array([6, -6, 4, 3, 2, 1.5, 1, 0.5], np.float32) * np.float32(G)
    assert np.array_equal(oracle.quant_nvfp4(y, G)[1], y / np.float32(G))


def test_nvfp4_dequant_and_ffn_closed_form():
    """Weights e2m1 code 2 (1.0) with scale code 0x38 (1.0) and tensor scale 1:
    every weight is 1; with x quantising to itself the FFN has a closed form."""
    words = np.full((3, 4), 0x22222222, np.uint32)               # K = 32
    W = oracle.dequantize_nvfp4(words, np.full((3, 2), 0x38, np.uint8))
    assert np.array_equal(W, np.ones((3, 32), np.float32))
    E, H, I = 2, 32, 16
    wt = {"w13_codes": np.full((E, 2 * I, H // 8), 0x22222222, np.uint32),
          "w13_scales": np.full((E, 2 * I, H // 16), 0x38, np.uint8), "w13_gscale": np.ones(E, np.float32),
          "w2_codes": np.full((E, H, I // 8), 0x22222222, np.uint32),
          "w2_scales": np.full((E, H, I // 16), 0x38, np.uint8), "w2_gscale": np.ones(E, np.float32)}
    G = 2.0 ** -8
    x = np.zeros((1, H), np.float32)
    x[0, :2] = np.float32(6 * G)                                 # groups quantise to themselves
    off = np.array([0, 1, 1], np.int32)
    y = oracle.expert_ffn_nvfp4(_bf16(x), off, np.array([0], np.int32), 1, wt, I, G, G)
    S = 12 * G
    h = S / (1 + np.exp(-S)) * S
    _, hq = oracle.quant_nvfp4(np.full((1, I), h, np.float32), G)
    assert np.allclose(y[0], hq.sum() * G * np.ones(H), rtol=1e-6)


def test_dequant_exact_against_integer_arithmetic():
    """(q - z) * s is exact: compare with exact rationals."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    w = rng.integers(0, 2**32, size=(2, 16), dtype=np.uint32)       # K = 256 at 2 bits
    s = _bf16(np.abs(rng.standard_normal((2, 2))) * 0.05)
    z = rng.integers(1, 3, size=(2, 2), dtype=np.uint8)
    W = oracle.dequantize(w, s, z, 2)
    sf = oracle.bf16_to_f32(s)
    for n in range(2):
        for kk in range(0, 256, 37):
            word = int(w[n, kk // 16])
            u = (word >> (2 * (kk % 16))) & 3
            exact = Fraction(u - int(z[n, kk // 128])) * Fraction(float(sf[n, kk // 128]))
            assert Fraction(float(W[n, kk])) == exact


# ------------------------------------------------------------------ O1 router
def _golden_router():
    cases = []
    for line in open(os.path.join(GOLDEN, "router_order.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        name, xs, ws, bias, exp, _why = [p.strip() for p in line.split("|")]
        parse = lambda s: [(int(a), float(b)) for a, b in (t.split(":") for t in s.split())]
        cases.append((name, parse(xs), parse(ws), float(bias), float(exp)))
    return cases


def test_router_order_golden():
    cases = _golden_router()
    assert len(cases) >= 5
    H = 256
    for name, xs, ws, bias, exp in cases:
        x = np.zeros((1, H), np.float32)
        w = np.zeros((1, H), np.float32)
        for h, v in xs:
            x[0, h] = v
        for h, v in ws:
            w[0, h] = v
        l = oracle.router_logits(_bf16(x), _bf16(w), np.array([bias], np.float32))
        assert float(l[0, 0]) == exp, name


def test_router_integer_inputs_exact():
    """With small integers every partial sum is exact: logits equal the integer dot."""
    rng = np.random.default_rng(2)
    T, E, H = 3, 5, 512
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-8, 9, size=(E, H))
    l = oracle.router_logits(_bf16(xi), _bf16(wi))
    exact = xi @ wi.T
    assert np.array_equal(l.astype(np.int64), exact)
    assert np.array_equal(l, exact.astype(np.float32))


def test_router_within_float32_error_bound_of_exact():
    """Against the exact dot (float64 of exact products) within the order's bound."""
    rng = np.random.default_rng(9)
    T, E, H = 4, 16, 4096
    x = _bf16(rng.standard_normal((T, H)))
    w = _bf16(rng.standard_normal((E, H)) * 0.02)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    absum = np.abs(xf) @ np.abs(wf).T
    l = oracle.router_logits(x, w)
    depth = H // 64 + 6                       # adds along any path of the order
    bound = depth * 2.0**-24 * absum * 1.01
    assert np.all(np.abs(l - exact) <= bound)
    # and it is not trivially exact: some logits differ from the float64 value
    assert np.any(l != exact.astype(np.float32))


def test_router_transposition_pinned():
    """Row e of W_r scores expert e: a one-hot x picks column h of W_r."""
    E, H = 6, 128
    w = np.arange(E * H, dtype=np.float32).reshape(E, H) % 7 - 3
    x = np.zeros((1, H), np.float32)
    x[0, 37] = 1.0
    l = oracle.router_logits(_bf16(x), _bf16(w))
    assert l[0].tolist() == w[:, 37].tolist()


# ------------------------------------------------------------------ O2/O3 top-k, softmax
def _brute_topk(l, k):
    """Rank counting: expert e is beaten by f if l_f > l_e or (l_f == l_e and f < e)."""
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        for e in range(E):
            rank = sum(1 for f in range(E) if l[t, f] > l[t, e] or (l[t, f] == l[t, e] and f < e))
            if rank < k:
                ids[t, rank] = e
    return ids


def test_topk_brute_force_random_and_ties():
    rng = np.random.default_rng(4)
    for E, k in [(8, 2), (8, 8), (16, 5), (7, 1)]:
        l = rng.standard_normal((6, E)).astype(np.float32)
        l[0, :] = 1.0                                 # all tied
        l[1, ::2] = l[1, 1]                           # partial ties
        l[2, 3] = l[2, 5] = l[2].max() + 1            # tie at the top
        ids, _ = oracle.topk_softmax(l, k)
        assert np.array_equal(ids, _brute_topk(l, k))


def test_topk_ties_from_duplicate_router_rows_pick_lower_index():
    rng = np.random.default_rng(6)
    H, E = 256, 8
    w = rng.standard_normal((E, H)).astype(np.float32) * 0.02
    w[5] = w[2]                                        # identical rows -> identical logits
    w[6] = w[2]
    x = _bf16(rng.standard_normal((3, H)))
    l = oracle.router_logits(x, _bf16(w))
    assert np.all(l[:, 5] == l[:, 2]) and np.all(l[:, 6] == l[:, 2])
    ids, _ = oracle.topk_softmax(l, E)
    for t in range(3):
        pos = {int(e): i for i, e in enumerate(ids[t])}
        assert pos[2] < pos[5] < pos[6]


def test_softmax_closed_forms():
    l = np.array([[2.0, 0.5, -1.0, 0.25]], np.float32)
    ids, g = oracle.topk_softmax(l, 1)
    assert ids.tolist() == [[0]] and g.tolist() == [[1.0]]
    ids, g = oracle.topk_softmax(l, 2)
    assert ids.tolist() == [[0, 1]]
    assert abs(g[0, 0] - 1.0 / (1.0 + math.exp(0.5 - 2.0))) < 1e-7
    assert abs(g[0, 1] - 1.0 / (1.0 + math.exp(2.0 - 0.5))) < 1e-7


def test_softmax_invariants():
    rng = np.random.default_rng(8)
    l = (rng.standard_normal((50, 32)) * 3).astype(np.float32)
    ids, g = oracle.topk_softmax(l, 8)
    assert np.all(np.abs(g.astype(np.float64).sum(1) - 1.0) < 1e-6)
    assert np.all(np.diff(g, axis=1) <= 0)            # slots in descending logit order
    assert np.all(g > 0)


# ------------------------------------------------------------------ O4 permutation
def _brute_positions(flat):
    n = len(flat)
    return np.array([sum(1 for r2 in range(n) if (flat[r2], r2) < (flat[r], r)) for r in range(n)])


@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (9, 3, 5), (1, 8, 256), (16, 8, 12), (3, 1, 1)])
def test_permutation_brute_force(T, k, E):
    rng = np.random.default_rng(T * 100 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, sr, rp, act = oracle.permute(ids, E)
    flat = ids.ravel()
    pos = _brute_positions(flat.tolist())
    assert np.array_equal(rp, pos)
    assert np.array_equal(sr[pos], np.arange(T * k))
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
    for e in range(E):
        rows = sr[off[e]:off[e + 1]]
        assert np.all(flat[rows] == e) and np.all(np.diff(rows) > 0)
    A = act[0]
    assert A == len(set(flat.tolist()))
    assert act[1:1 + A].tolist() == sorted(set(flat.tolist()))
    assert np.all(act[1 + A:] == -1)
    assert act.size == 1 + min(E, T * k)


# ------------------------------------------------------------------ O7/O8 FFN + combine
def _tiny(bits=4, **kw):
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", **kw)
    if bits == 6:
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", bits=6, **kw)
    elif bits == 2:
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", bits=2, scale_sigma=0.05, **kw)
    elif bits == 8:
        sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", bits=8, scale_sigma=0.0015, **kw)
    return workload.make_layer_inputs(sp)


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 128), (4, 32), (8, 128), (8, 32), (6, 128)])
def test_ffn_all_equal_weights_closed_form(bits, group):
    """Every weight = c: A_n = c*S (S = sum of x), h = silu(cS)*cS, y = I*c*h for all rows."""
    inp = _tiny(bits, group=group)
    sp = inp.spec
    E, H, I = sp.E, sp.H, sp.I
    wt = dict(inp.weights)
    if bits == 4:
        word, c = 0x99999999, 1.0                     # q = 1
        z13 = z2 = None
    elif bits == 8:
        word, c = 0x7F7F7F7F, -1.0                    # q = -1
    elif bits == 6:
        word, c = None, 1.0                           # e2m3 code 8 = 1.0 (tests/golden/fp6_e2m3.txt)
    else:
        word, c = 0xFFFFFFFF, 2.0                     # u = 3, z = 1 -> 2
        wt["w13_zeros"] = np.ones_like(wt["w13_zeros"])
        wt["w2_zeros"] = np.ones_like(wt["w2_zeros"])
    if bits == 6:   # the hand-packed row of sixteen code-8 fields, repeated
        trip = np.array([0x08208208, 0x82082082, 0x20820820], np.uint32)
        for key in ("w13_codes", "w2_codes"):
            shp = wt[key].shape
            wt[key] = np.ascontiguousarray(np.broadcast_to(np.tile(trip, shp[-1] // 3), shp))
        one = np.uint16(0x3C00)                       # fp16 1.0
        wt["w13_scales"] = np.full(wt["w13_scales"].shape, one, np.uint16)
        wt["w2_scales"] = np.full(wt["w2_scales"].shape, one, np.uint16)
    else:
        wt["w13_codes"] = np.full_like(wt["w13_codes"], word)
        wt["w2_codes"] = np.full_like(wt["w2_codes"], word)
        wt["w13_scales"] = _bf16(np.ones(wt["w13_scales"].shape))
        wt["w2_scales"] = _bf16(np.ones(wt["w2_scales"].shape))
    out = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, wt, sp.k, bits, I, group=group)
    xf = oracle.bf16_to_f32(inp.x).astype(np.float64)
    S = c * xf.sum(1)
    hval = S / (1 + np.exp(-S)) * S
    expect = (I * c * hval)[:, None] * np.ones((1, H))
    assert oracle.rel_fro(out["y"], expect) < 1e-5
    # each sorted row holds its token's value
    tok = out["sorted_rows"] // sp.k
    assert oracle.rel_fro(out["y_perm"], expect[tok]) < 1e-5


def test_ffn_one_hot_input_reads_one_weight_column():
    """x = e_j gives A[n] = W13[n, j] (orientation A = X W^T, gate rows first)."""
    inp = _tiny(4)
    sp = inp.spec
    I = sp.I
    j = 77
    x = np.zeros((1, sp.H), np.float32)
    x[0, j] = 1.0
    e = 3
    off = np.array([0] * (e + 1) + [1] * (sp.E - e), np.int32)
    y = oracle.expert_ffn(_bf16(x), off, np.array([0], np.int32), 1, inp.weights, 4, I, experts=[e])
    # expected from the bits directly
    codes = inp.weights["w13_codes"][e]
    sc = oracle.bf16_to_f32(inp.weights["w13_scales"][e])
    a = np.empty(2 * I)
    for n in range(2 * I):
        u = (int(codes[n, j // 8]) >> (4 * (j % 8))) & 15
        a[n] = (u - 8) * float(sc[n, j // 128])
    h = a[:I] / (1 + np.exp(-a[:I])) * a[I:]
    W2 = oracle.dequantize(inp.weights["w2_codes"][e], inp.weights["w2_scales"][e], None, 4).astype(np.float64)
    assert oracle.rel_fro(y[0], W2 @ h) < 1e-5


@pytest.mark.parametrize("bits", [4, 8])
def test_ffn_one_hot_input_group32_reads_bytes_directly(bits):
    """Group 32: x = e_j gives A[n] = (field - offset) * s[n, j // 32], read from the bits."""
    inp = _tiny(bits, group=32)
    sp = inp.spec
    I, P = sp.I, 32 // bits
    e = 5
    off = np.array([0] * (e + 1) + [1] * (sp.E - e), np.int32)
    codes = inp.weights["w13_codes"][e]
    sc = oracle.bf16_to_f32(inp.weights["w13_scales"][e])
    W2 = oracle.dequantize(inp.weights["w2_codes"][e], inp.weights["w2_scales"][e], None, bits,
                           group=32).astype(np.float64)
    for j in (0, 31, 32, 95, 200):
        x = np.zeros((1, sp.H), np.float32)
        x[0, j] = 1.0
        y = oracle.expert_ffn(_bf16(x), off, np.array([0], np.int32), 1, inp.weights, bits, I, experts=[e],
                              group=32)
        a = np.empty(2 * I)
        for n in range(2 * I):
            u = (int(codes[n, j // P]) >> (bits * (j % P))) & ((1 << bits) - 1)
            a[n] = (u - (1 << (bits - 1))) * float(sc[n, j // 32])
        h = a[:I] / (1 + np.exp(-a[:I])) * a[I:]
        assert oracle.rel_fro(y[0], W2 @ h) < 1e-5


@pytest.mark.parametrize("bits", [4, 2])
def test_dense_equivalence_all_experts_selected(bits):
    """k = E: the routed layer equals sum_e softmax(l)_e FFN_e(x) computed densely."""
    inp = _tiny(bits, k=8)
    sp = inp.spec
    out = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, bits, sp.I)
    xf = oracle.bf16_to_f32(inp.x).astype(np.float64)
    l = out["logits"].astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    y = np.zeros((sp.T, sp.H))
    for e in range(sp.E):
        z13 = inp.weights.get("w13_zeros")
        z2 = inp.weights.get("w2_zeros")
        W13 = oracle.dequantize(inp.weights["w13_codes"][e], inp.weights["w13_scales"][e],
                                None if z13 is None else z13[e], bits).astype(np.float64)
        W2 = oracle.dequantize(inp.weights["w2_codes"][e], inp.weights["w2_scales"][e],
                               None if z2 is None else z2[e], bits).astype(np.float64)
        A = xf @ W13.T
        h = A[:, :sp.I] / (1 + np.exp(-A[:, :sp.I])) * A[:, sp.I:]
        y += p[:, e:e + 1] * (h @ W2.T)
    assert oracle.rel_fro(out["y"], y) < 1e-5


@pytest.mark.parametrize("bits,group", [(4, 128), (2, 128), (4, 32), (8, 128), (8, 32), (6, 128)])
def test_float32_oracle_close_to_float64(bits, group):
    inp = _tiny(bits, group=group)
    sp = inp.spec
    o32 = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, bits, sp.I, group=group)
    o64 = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, bits, sp.I,
                           dtype=np.float64, group=group)
    assert np.array_equal(o32["ids"], o64["ids"])
    assert oracle.rel_fro(o32["y"], o64["y"]) < 1e-5


def test_per_token_runs_equal_batched_run():
    inp = _tiny(4)
    sp = inp.spec
    full = oracle.moe_layer(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, 4, sp.I)
    for t in range(sp.T):
        one = oracle.moe_layer_tokens(inp.x, inp.w_router, inp.logit_bias, inp.weights, sp.k, 4, sp.I, [t])
        assert np.array_equal(one["ids"][0], full["ids"][t])
        assert np.allclose(one["y"][0], full["y"][t], rtol=1e-5, atol=1e-6)


def test_combine_weights_rows_by_gates():
    """Combine with one-hot gates returns the selected row exactly."""
    y_perm = np.arange(12, dtype=np.float32).reshape(6, 2)
    row_pos = np.array([4, 1, 0, 5, 2, 3], np.int32)          # T=3, k=2
    gates = np.array([[1, 0], [0, 1], [0.25, 0.75]], np.float32)
    y = oracle.combine(y_perm, row_pos, gates)
    assert y[0].tolist() == y_perm[4].tolist()
    assert y[1].tolist() == y_perm[5].tolist()
    assert np.allclose(y[2], 0.25 * y_perm[2] + 0.75 * y_perm[3])


# ------------------------------------------------------------------ helpers the parity bars rest on
def test_rel_fro_hand_computed_values():
    """||a - ref||_F / ||ref||_F on hand-computed cases: the right numerator, the
    reference's norm as denominator (not a's), Frobenius over every element
    (not a per-row or spectral norm)."""
    ref = np.array([6.0, 8.0])                                   # norm 10
    assert oracle.rel_fro(np.array([9.0, 12.0]), ref) == 0.5     # diff (3, 4): norm 5
    assert oracle.rel_fro(ref, ref) == 0.0
    assert abs(oracle.rel_fro(np.array([6.0, 8.0]), np.array([9.0, 12.0])) - 5.0 / 15.0) < 1e-15
    # matrix: diff = identity (Frobenius sqrt 2, spectral 1), ref Frobenius 2
    r2 = np.array([[2.0, 0.0], [0.0, 0.0]])
    a2 = r2 + np.eye(2)
    assert abs(oracle.rel_fro(a2, r2) - math.sqrt(2.0) / 2.0) < 1e-15
    # float32 inputs are measured in float64: a 1-ulp difference is not lost
    one = np.float32(1.0)
    assert oracle.rel_fro(np.array([np.nextafter(one, np.float32(2))], np.float32), np.array([one])) == 2.0 ** -23


def test_bf16_bits_and_silu_closed_forms():
    """bf16 bits are the top half of float32; silu(v) = v * sigmoid(v)."""
    assert oracle.bf16_to_f32(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049], np.uint16)).tolist() == \
        [1.0, -2.0, 0.0, -0.0, 3.140625]
    v = np.array([0.0, math.log(3.0), -math.log(3.0)], np.float32)
    got = oracle.silu(v).astype(np.float64)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * math.log(3.0)) < 1e-6 and abs(got[2] + 0.25 * math.log(3.0)) < 1e-6


def test_router_token_blocks_do_not_change_bits():
    """Tokens are independent: a batch crossing the oracle's token blocks gives
    each token's logits bit for bit as a call with that token alone."""
    rng = np.random.default_rng(17)
    T, E, H = 37, 9, 256
    x = _bf16(rng.standard_normal((T, H)))
    w = _bf16(rng.standard_normal((E, H)) * 0.05)
    b = (rng.standard_normal(E) * 0.01).astype(np.float32)
    full = oracle.router_logits(x, w, b)
    for t in (0, 15, 16, 17, 36):
        one = oracle.router_logits(x[t:t + 1], w, b)
        assert np.array_equal(one[0].view(np.uint32), full[t].view(np.uint32)), t


# ------------------------------------------------------------------ NVFP4 field order, scale placement, tensor scales
def test_nvfp4_nibble_order_distinct_fields():
    """Field i of word w is K index 8w + i, least significant nibble first:
    words with eight distinct nibbles fix the order."""
    words = np.array([[0x76543210, 0xFEDCBA98]], np.uint32)
    assert oracle.unpack_e2m1_fields(words).tolist() == [list(range(16))]
    # and the value table applied in that order: codes 0..7 positive, 8..15 their negatives
    v = oracle.e2m1_value(oracle.unpack_e2m1_fields(words))[0]
    assert v.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                          -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_nvfp4_group_scale_lands_on_its_own_16_columns():
    """A different E4M3 scale per group of 16 (and per row): each scale
    multiplies exactly its own 16 consecutive K (np.tile or a transposed
    scale array would not)."""
    words = np.full((2, 8), 0x22222222, np.uint32)               # every code 2 = 1.0, K = 64
    sc = np.array([[0x38, 0x40, 0x30, 0x48],                     # 1, 2, 0.5, 4
                   [0x3C, 0x28, 0x01, 0x7E]], np.uint8)          # 1.5, 0.25, 2^-9, 448
    W = oracle.dequantize_nvfp4(words, sc)
    exp = np.array([[1.0] * 16 + [2.0] * 16 + [0.5] * 16 + [4.0] * 16,
                    [1.5] * 16 + [0.25] * 16 + [2.0 ** -9] * 16 + [448.0] * 16], np.float32)
    assert np.array_equal(W, exp)


def test_nvfp4_ffn_tensor_scales_closed_form():
    """G_x != G_h and w13_gscale != w2_gscale (powers of two, different per
    expert): the closed form below changes by a factor of 8 or more if any
    two of them are exchanged.  Every weight is 1 (code 2, scale 1.0); the
    token's first two values are 6 G_x, so its quantised row is (6, 6, 0...)
    (scale E4M3(1) = 1), A = 12 G_x g13[e] on every output, h = silu(A) A on
    all I values, which quantise to 6 s with s = E4M3(h / (6 G_h)) (within
    2^-4 of h / (6 G_h), and on the E4M3 grid), and y = I * 6 s * G_h * g2[e]."""
    E, H, I = 2, 32, 16
    Gx, Gh = 2.0 ** -8, 2.0 ** -5
    g13 = np.array([2.0, 8.0], np.float32)
    g2 = np.array([0.25, 16.0], np.float32)
    wt = {"w13_codes": np.full((E, 2 * I, H // 8), 0x22222222, np.uint32),
          "w13_scales": np.full((E, 2 * I, H // 16), 0x38, np.uint8), "w13_gscale": g13,
          "w2_codes": np.full((E, H, I // 8), 0x22222222, np.uint32),
          "w2_scales": np.full((E, H, I // 16), 0x38, np.uint8), "w2_gscale": g2}
    x = np.zeros((1, H), np.float32)
    x[0, :2] = np.float32(6 * Gx)
    grid8 = set(oracle.e4m3_value(np.arange(0x7F)).tolist())
    for e in range(E):
        off = np.array([0] * (e + 1) + [1] * (E - e), np.int32)
        y = oracle.expert_ffn_nvfp4(_bf16(x), off, np.array([0], np.int32), 1, wt, I, Gx, Gh)[0].astype(np.float64)
        A = 12.0 * Gx * float(g13[e])
        h = A / (1.0 + math.exp(-A)) * A
        s = y[0] / (I * 6.0 * Gh * float(g2[e]))                  # the group scale the quantiser chose
        assert np.all(y == y[0])
        assert s in grid8, s
        assert abs(s / (h / (6.0 * Gh)) - 1.0) <= 2.0 ** -4, (e, s, h)


def test_nvfp4_dense_equivalence_all_experts_selected():
    """k = E with NVFP4 experts: the routed layer equals sum_e softmax(l)_e
    FFN_e(x), each FFN_e written out densely from the format's definition
    (quantise x, dequantise both matrices, tensor scales after the products)."""
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", group=16, k=8)
    inp = workload.make_layer_inputs(sp)
    out = oracle.moe_layer_nvfp4(inp.x, inp.w_router, None, inp.weights, sp.k, sp.I, sp.nv_gx, sp.nv_gh)
    xf = oracle.bf16_to_f32(inp.x)
    l = out["logits"].astype(np.float64)
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    _, xq = oracle.quant_nvfp4(xf, sp.nv_gx)
    y = np.zeros((sp.T, sp.H))
    w = inp.weights
    for e in range(sp.E):
        W13 = oracle.dequantize_nvfp4(w["w13_codes"][e], w["w13_scales"][e]).astype(np.float64)
        W2 = oracle.dequantize_nvfp4(w["w2_codes"][e], w["w2_scales"][e]).astype(np.float64)
        A = (xq.astype(np.float64) @ W13.T) * (sp.nv_gx * float(w["w13_gscale"][e]))
        h = (A[:, :sp.I] / (1 + np.exp(-A[:, :sp.I])) * A[:, sp.I:]).astype(np.float32)
        _, hq = oracle.quant_nvfp4(h, sp.nv_gh)
        y += p[:, e:e + 1] * ((hq.astype(np.float64) @ W2.T) * (sp.nv_gh * float(w["w2_gscale"][e])))
    assert oracle.rel_fro(out["y"], y) < 1e-4
