"""CPU oracle for the routed-expert MoE layer with low-bit (INT4 / 2-bit / INT8 / FP6) experts.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference that the
GPU library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library's product path never
does.  It shares no code with the GPU path: it reads the same numpy input
arrays (from the ``workload`` generator) and nothing else.

What it computes, step by step (the numbering is used by the tests):

O1  router logits in one fixed float32 summation order;
O2  top-k experts per token, ties to the lower expert index;
O3  softmax over the k selected logits (float64, stored as float32);
O4  stable counting-sort permutation of the T*k (token, slot) rows by expert;
O5  unpacking of the packed code words;
O6  dequantisation w = (q - z) * s per K group (128 wide, or 32);
O7  per-expert FFN: gate_up matmul, SwiGLU, down matmul (float32);
O8  weighted combine of each token's k expert outputs (float32).

Sources.  The weight formats come from the pages: INT4 symmetric group-128
weight-only experts with 16-bit activations (page "Qwen3.8-Flash-Next on 2x RTX
3090", storage-format table; page "Qwen3.8-Flash-Next on dual RTX 3090: W4A16 +
FP8 PLE + MTP3", "Composition"), and 2-bit group-128 GPTQ-style experts with 16
codes per 32-bit word along K (page "Qwen3.8-Flash-Next on one 24 GB GPU",
"What the patch does" and "Hardware and software requirements").  Two more
formats take the same path with other group sizes and widths: INT4 symmetric
with group 32 (the draft-layer experts of page "Qwen3.8-Flash-Next on 2x RTX
3090", storage-format table, and of page "Qwen3.8-Flash-Next on dual RTX 3090:
W4A16 + FP8 PLE + MTP3", "Composition"), and INT8 symmetric with codes
-127..127 and group 128 or 32 (page "Qwen3.8-Flash-Next on one 24 GB GPU",
"What the patch does": dense projections re-packed to INT8 g128; page
"Qwen3.8-Flash-Next FP6-INT8", "Precision map" and "Kernel-level
verification": an int8 g32 tier).  FP6 experts hold e2m3 codes (sign, 2
exponent bits with bias 1, 3 mantissa bits; values up to 7.5, exact in bf16)
with fp16 scales (same page: fp6 e2m3 routed experts, every one of the 64
codes checked exactly, fp16 scales); here one scale per 128 K.  The pages fix
activations at bf16 with float32 accumulation (page "Qwen3.8-Flash-Next
FP6-INT8", "Precision map"), so the oracle accumulates in float32.  They keep
the router in 16-bit precision because near-tied logits flip routing under
small perturbations (same page, "Precision map"); that is why O1 fixes one
summation order.  The pages do not describe the MoE block itself (top-k
softmax, SwiGLU, gate/up row order, combine); those steps follow the plainest
reading of the layer this library implements, and every such reading is listed
with the design notes.

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, hand-derived golden values, brute force or invariants.
"""
from __future__ import annotations

import os

# Single-threaded BLAS for a reproducible, honest single-core baseline.
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, "1")

import numpy as np  # noqa: E402

GROUP = 128
SLICES = 64  # O1: number of contiguous K slices of the router dot product


# ---------------------------------------------------------------- helpers
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bits (uint16) -> float32, exactly (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- O5, O6
FP6 = 6  # the ``bits`` value that selects fp6 e2m3 codes with fp16 scales


def unpack_fp6_fields(words: np.ndarray) -> np.ndarray:
    """O5 (FP6): words [..., 3K/16] -> 6-bit codes [..., K] (uint8).

    A row's codes form one little-endian bit stream: code k occupies bits
    [6k, 6k+6) of the row (bit b of the stream is bit b % 32 of word b // 32),
    16 codes per 3 words.
    """
    w = np.ascontiguousarray(words, dtype=np.uint32)
    nw = w.shape[-1]
    if nw % 3:
        raise ValueError("FP6 rows hold a multiple of 3 words")
    K = nw * 32 // 6
    k = np.arange(K)
    lo_word, lo_bit = (6 * k) // 32, (6 * k) % 32
    w64 = w.astype(np.uint64)
    nxt = np.concatenate([w64[..., 1:], np.zeros(w64.shape[:-1] + (1,), np.uint64)], axis=-1)
    pair = w64 | (nxt << np.uint64(32))                       # word i and i+1 as one 64-bit value
    return ((pair[..., lo_word] >> lo_bit.astype(np.uint64)) & np.uint64(63)).astype(np.uint8)


def e2m3_value(codes: np.ndarray) -> np.ndarray:
    """The value of fp6 e2m3 codes: bit 5 sign, bits 4..3 exponent e (bias 1),
    bits 2..0 mantissa m; e = 0 is subnormal (m / 8), otherwise
    2^(e-1) * (1 + m/8).  No infinities or NaNs."""
    c = np.asarray(codes, dtype=np.int64)
    sgn = np.where(c & 32, -1.0, 1.0)
    e, m = (c >> 3) & 3, c & 7
    mag = np.where(e == 0, m / 8.0, np.exp2(e - 1.0) * (1.0 + m / 8.0))
    return (sgn * mag).astype(np.float32)


def unpack_codes(words: np.ndarray, bits: int) -> np.ndarray:
    """O5: packed words [..., K/P] -> signed integer codes q [..., K] (int8).

    Field i of word kw (bits [b*i, b*i+b), least significant first) holds the
    code for K index P*kw + i, P = 32/b.  INT4 fields store q + 8 (offset
    binary), so q = field - 8 spans [-8, 7]; INT8 fields store q + 128, so
    q = field - 128 (the format uses -127..127); 2-bit fields store q in {0..3}
    directly and the zero-point is subtracted at dequantisation.
    """
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    w = np.ascontiguousarray(words, dtype=np.uint32)
    P = 32 // bits
    mask = np.uint32((1 << bits) - 1)
    fields = np.empty(w.shape + (P,), dtype=np.int16)
    for i in range(P):
        fields[..., i] = ((w >> np.uint32(bits * i)) & mask).astype(np.int16)
    q = fields.reshape(w.shape[:-1] + (w.shape[-1] * P,))
    if bits == 4:
        q = q - 8
    elif bits == 8:
        q = q - 128
    return q.astype(np.int8)


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of unpack_codes: signed codes [..., K] -> words [..., K/P]."""
    q = np.asarray(q, dtype=np.int16)
    P = 32 // bits
    if q.shape[-1] % P:
        raise ValueError("K must be a multiple of codes-per-word")
    u = q + {4: 8, 8: 128}.get(bits, 0)
    if u.min(initial=0) < 0 or u.max(initial=0) >= (1 << bits):
        raise ValueError("code out of range")
    u = u.astype(np.uint32).reshape(q.shape[:-1] + (q.shape[-1] // P, P))
    w = np.zeros(u.shape[:-1], dtype=np.uint32)
    for i in range(P):
        w |= u[..., i] << np.uint32(bits * i)
    return w


def dequantize(words: np.ndarray, scales: np.ndarray, zeros, bits: int, group: int = GROUP) -> np.ndarray:
    """O6: one expert matrix [N, K/P] words -> float32 weights [N, K].

    W[n, k] = (q[n, k] - z[n, k // G]) * s[n, k // G] for group size G, with
    z = 0 for the symmetric INT4 and INT8 formats.  (q - z) is an integer of at
    most 8 bits and s a bf16 value (8 significant bits), so the product is
    exact in float32.  FP6 (bits = 6): W = e2m3(code) * s with s an fp16
    value; 4 and 11 significant bits, again exact in float32.
    """
    if bits == FP6:
        v = e2m3_value(unpack_fp6_fields(words))                # [N, K]
        N, K = v.shape
        if K % group:
            raise ValueError("K must be a multiple of the group size")
        s = np.ascontiguousarray(scales, dtype=np.uint16).view(np.float16).astype(np.float32).reshape(N, K // group)
        return (v * np.repeat(s, group, axis=1)).astype(np.float32)
    q = unpack_codes(words, bits).astype(np.float32)           # [N, K]
    N, K = q.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    s = bf16_to_f32(scales).reshape(N, K // group)
    s_full = np.repeat(s, group, axis=1)                        # [N, K]
    if zeros is None:
        z_full = np.zeros_like(q)
    else:
        z_full = np.repeat(np.asarray(zeros, dtype=np.float32).reshape(N, K // group), group, axis=1)
    return ((q - z_full) * s_full).astype(np.float32)


# ---------------------------------------------------------------- O1
def router_logits(x: np.ndarray, w_router: np.ndarray, bias=None) -> np.ndarray:
    """O1: logits l[t, e] = sum_h x[t, h] * W_r[e, h] (+ b[e]) in float32.

    The order of the float32 additions is fixed, because routing must come out
    identical on every implementation and near-tied logits otherwise flip:
    split h into 64 contiguous slices of H/64 elements; within a slice add the
    products to a running sum that starts at 0, in ascending h; then add the
    64 slice sums as a balanced binary tree in index order ((s0+s1), (s2+s3),
    ..., then pairs of those, six levels); finally add the bias.  Products of
    two bf16 values are exact in float32, so the only roundings are these adds.
    """
    xf = bf16_to_f32(x)
    wf = bf16_to_f32(w_router)
    T, H = xf.shape
    E = wf.shape[0]
    if H % SLICES:
        raise ValueError("H must be a multiple of 64")
    L = H // SLICES
    ws = np.ascontiguousarray(wf.reshape(E, SLICES, L).transpose(2, 0, 1))      # [L, E, 64]: element i of each slice
    logits = np.empty((T, E), dtype=np.float32)
    # Tokens are independent, so they are taken a few at a time (the arrays
    # then stay in cache); every logit sees the same operations in the same
    # order whatever the block size.
    for t0 in range(0, T, _ROUTER_TOKENS):
        xs = np.ascontiguousarray(xf[t0:t0 + _ROUTER_TOKENS].reshape(-1, SLICES, L).transpose(2, 0, 1))  # [L, n, 64]
        n = xs.shape[1]
        part = np.zeros((n, E, SLICES), dtype=np.float32)
        prod = np.empty_like(part)
        for i in range(L):                                      # ascending h in each slice
            np.multiply(xs[i][:, None, :], ws[i][None, :, :], out=prod)   # float32 product (exact)
            np.add(part, prod, out=part)                        # float32 add
        while part.shape[-1] > 1:                               # pairwise tree
            part = part[..., 0::2] + part[..., 1::2]
        logits[t0:t0 + n] = part[..., 0]
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float32)[None, :]
    return logits.astype(np.float32)


_ROUTER_TOKENS = 16  # tokens per block of the router loop (speed only)


# ---------------------------------------------------------------- O2, O3
def topk_softmax(logits: np.ndarray, k: int):
    """O2 + O3: ids [T, k] int32 and gates [T, k] float32.

    The k selected experts are the first k in the order (logit descending,
    expert index ascending) and are listed in that order.  The gates are the
    softmax of the k selected logits, computed in float64.
    """
    l = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l)):
        raise ValueError("non-finite logit")
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    e_idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((e_idx, -l[t].astype(np.float64)))  # primary: -l, secondary: e
        sel = order[:k]
        ids[t] = sel
        v = l[t, sel].astype(np.float64)
        ex = np.exp(v - v[0])                                    # v[0] is the maximum
        gates[t] = (ex / ex.sum()).astype(np.float32)
    return ids, gates


# ---------------------------------------------------------------- O4
def permute(ids: np.ndarray, E: int):
    """O4: group the T*k rows r = t*k + j by expert, keeping r ascending within an expert.

    Returns expert_offsets [E+1], sorted_rows [T*k] (row r at each sorted
    position), row_pos [T*k] (sorted position of each row r) and active
    [1 + min(E, T*k)] (the number A of experts with rows, then their ids
    ascending, then -1 padding).
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    n = flat.size
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_rows = np.argsort(flat, kind="stable").astype(np.int32)
    row_pos = np.empty(n, dtype=np.int32)
    row_pos[sorted_rows] = np.arange(n, dtype=np.int32)
    act = np.nonzero(counts)[0].astype(np.int32)
    active = np.full(1 + min(E, n), -1, dtype=np.int32)
    active[0] = act.size
    active[1:1 + act.size] = act
    return offsets, sorted_rows, row_pos, active


# ---------------------------------------------------------------- O7
def silu(a: np.ndarray) -> np.ndarray:
    return a / (np.float32(1.0) + np.exp(-a))


def expert_ffn(x, offsets, sorted_rows, k: int, weights: dict, bits: int, I: int,
               experts=None, dtype=np.float32, group: int = GROUP) -> np.ndarray:
    """O7: y_perm [T*k, H]: the expert FFN of every row, in sorted order.

    For expert e with rows R = sorted_rows[o_e : o_(e+1)] (tokens R // k):
        A = X_e @ W13_e^T                 (gate_up, [n_e, 2I])
        h = silu(A[:, :I]) * A[:, I:]     (rows [0, I) of W13 are gate, [I, 2I) up)
        Y = h @ W2_e^T                    ([n_e, H])
    All intermediates stay in ``dtype`` (float32 by default).  ``experts``
    limits the work to a subset of experts (other rows are left as NaN).
    """
    xf = bf16_to_f32(x).astype(dtype)
    T, H = xf.shape
    E = offsets.size - 1
    y = np.full((sorted_rows.size, H), np.nan, dtype=dtype)
    zk13 = weights.get("w13_zeros")
    zk2 = weights.get("w2_zeros")
    for e in (range(E) if experts is None else experts):
        o0, o1 = int(offsets[e]), int(offsets[e + 1])
        if o1 == o0:
            continue
        toks = sorted_rows[o0:o1] // k
        Xe = xf[toks]
        W13 = dequantize(weights["w13_codes"][e], weights["w13_scales"][e],
                         None if zk13 is None else zk13[e], bits, group).astype(dtype)
        A = Xe @ W13.T
        h = silu(A[:, :I]) * A[:, I:]
        W2 = dequantize(weights["w2_codes"][e], weights["w2_scales"][e],
                        None if zk2 is None else zk2[e], bits, group).astype(dtype)
        y[o0:o1] = h @ W2.T
    return y


# ---------------------------------------------------------------- O8
def combine(y_perm: np.ndarray, row_pos: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """O8: y[t] = sum over j ascending of g[t, j] * y_perm[row_pos[t*k + j]]."""
    T, k = gates.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=y_perm.dtype)
    for j in range(k):
        y = y + gates[:, j:j + 1].astype(y_perm.dtype) * y_perm[row_pos[np.arange(T) * k + j]]
    return y


# ---------------------------------------------------------------- whole layer
def moe_layer(x, w_router, logit_bias, weights, k: int, bits: int, I: int, dtype=np.float32,
              group: int = GROUP) -> dict:
    """O1..O8 on one batch; returns every intermediate for element-wise checks."""
    E = w_router.shape[0]
    logits = router_logits(x, w_router, logit_bias)
    ids, gates = topk_softmax(logits, k)
    offsets, sorted_rows, row_pos, active = permute(ids, E)
    y_perm = expert_ffn(x, offsets, sorted_rows, k, weights, bits, I, dtype=dtype, group=group)
    y = combine(y_perm, row_pos, gates)
    return dict(logits=logits, ids=ids, gates=gates, offsets=offsets, sorted_rows=sorted_rows,
                row_pos=row_pos, active=active, y_perm=y_perm, y=y)


def moe_layer_tokens(x, w_router, logit_bias, weights, k: int, bits: int, I: int, tokens,
                     dtype=np.float32, group: int = GROUP) -> dict:
    """The layer output for a subset of tokens only (each token is independent).

    Used to check full-size runs on sampled tokens: routing of the sampled
    tokens, and their outputs, are computed from the same definitions.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    xs = np.asarray(x)[tokens]
    return moe_layer(xs, w_router, logit_bias, weights, k, bits, I, dtype=dtype, group=group)


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    """Relative Frobenius error ||a - ref|| / ||ref|| in float64."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / (den if den > 0 else 1.0))


# ---------------------------------------------------------------- NVFP4 (W4A4)
# Page "Qwen3.8-Flash-Next NVFP4", "Format": routed experts in NVFP4 W4A4, E2M1
# values in groups of 16.  The rest of the format is NVFP4's public
# definition, taken as the reading: each group of 16 consecutive K carries one
# FP8 E4M3 scale, a tensor carries one float32 scale, and activations are
# quantised the same way on the fly.  Every rounding below is to nearest,
# ties to even.
NVFP4_GROUP = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1: bit 3 sign, bits 2..1 exponent e (bias 1), bit 0 mantissa m;
    e = 0 is subnormal (m / 2), otherwise 2^(e-1) * (1 + m/2)."""
    c = np.asarray(codes, dtype=np.int64)
    sgn = np.where(c & 8, -1.0, 1.0)
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e == 0, m / 2.0, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return (sgn * mag).astype(np.float32)


def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (the finite codes): bit 7 sign, bits 6..3 exponent e (bias 7),
    bits 2..0 mantissa m; e = 0 is subnormal (m / 8 * 2^-6)."""
    c = np.asarray(codes, dtype=np.int64)
    sgn = np.where(c & 128, -1.0, 1.0)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, np.exp2(e - 7.0) * (1.0 + m / 8.0))
    return (sgn * mag).astype(np.float32)


def _round_to_grid(v: np.ndarray, min_exp: int, mbits: int, vmax: float) -> np.ndarray:
    """|v| rounded to a float grid with mbits mantissa bits whose smallest
    binade starts at 2^min_exp (below it the spacing stays 2^(min_exp-mbits)),
    ties to even, saturating at vmax; sign kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, min_exp)          # floor(log2 a), at least min_exp
    q = np.exp2(e - mbits)                   # spacing in that binade
    r = np.minimum(np.rint(a / q) * q, vmax)
    return np.where(v < 0, -r, r)


def round_e4m3(v):
    return _round_to_grid(v, -6, 3, E4M3_MAX).astype(np.float32)


def round_e2m1(v):
    return _round_to_grid(v, 0, 1, E2M1_MAX).astype(np.float32)


def quant_nvfp4(x: np.ndarray, gscale: float):
    """NVFP4 quantisation of float32 rows [..., K] with tensor scale G.

    Per group of 16: amax = max |x|; s = E4M3(amax / (6 G)); the codes are
    E2M1(x / (s G)) (all zero when s = 0).  Each step is one float32
    operation (6 G, then the division; s G, then the division), as written.
    Returns the group scales s [..., K/16] and the values q * s [..., K],
    both exact in float32 (and in bf16).
    """
    xf = np.asarray(x, dtype=np.float32)
    K = xf.shape[-1]
    g = xf.reshape(xf.shape[:-1] + (K // NVFP4_GROUP, NVFP4_GROUP))
    G = np.float32(gscale)
    amax = np.abs(g).max(axis=-1)
    s = round_e4m3(amax / (np.float32(6.0) * G))
    sg = (s * G).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(sg[..., None] > 0, g / sg[..., None], np.float32(0.0)).astype(np.float32)
    q = round_e2m1(t)
    return s, (q * s[..., None]).reshape(xf.shape).astype(np.float32)


def unpack_e2m1_fields(words: np.ndarray) -> np.ndarray:
    """NVFP4 weight words [..., K/8] -> 4-bit codes [..., K] (field i of word w is K index 8w + i)."""
    w = np.ascontiguousarray(words, dtype=np.uint32)
    f = np.stack([(w >> np.uint32(4 * i)) & np.uint32(15) for i in range(8)], axis=-1)
    return f.reshape(w.shape[:-1] + (w.shape[-1] * 8,)).astype(np.uint8)


def dequantize_nvfp4(words: np.ndarray, bscales: np.ndarray) -> np.ndarray:
    """One NVFP4 weight matrix without its tensor scale: e2m1(code) * e4m3(s) [N, K], exact."""
    v = e2m1_value(unpack_e2m1_fields(words))
    s = e4m3_value(bscales)
    return (v * np.repeat(s, NVFP4_GROUP, axis=-1)).astype(np.float32)


def expert_ffn_nvfp4(x, offsets, sorted_rows, k: int, weights: dict, I: int, x_gscale: float, h_gscale: float,
                     experts=None, dtype=np.float32) -> np.ndarray:
    """O7 for NVFP4 W4A4: y_perm [T*k, H].

    For expert e with rows R (tokens R // k):
        X' = NVFP4(x rows, G_x)                  (activation quantisation)
        A  = (X' W13'^T) * (G_x * G_w13[e])      (W' = e2m1 * e4m3 group scale)
        h  = silu(A[:, :I]) * A[:, I:]
        H' = NVFP4(h, G_h)
        Y  = (H' W2'^T) * (G_h * G_w2[e])
    """
    xf = bf16_to_f32(x).astype(np.float32)
    T, H = xf.shape
    E = offsets.size - 1
    y = np.full((sorted_rows.size, H), np.nan, dtype=dtype)
    gx, gh = np.float32(x_gscale), np.float32(h_gscale)
    for e in (range(E) if experts is None else experts):
        o0, o1 = int(offsets[e]), int(offsets[e + 1])
        if o1 == o0:
            continue
        _, Xq = quant_nvfp4(xf[sorted_rows[o0:o1] // k], gx)
        W13 = dequantize_nvfp4(weights["w13_codes"][e], weights["w13_scales"][e]).astype(dtype)
        A = (Xq.astype(dtype) @ W13.T) * dtype(gx * np.float32(weights["w13_gscale"][e]))
        h = (silu(A[:, :I]) * A[:, I:]).astype(np.float32)
        _, Hq = quant_nvfp4(h, gh)
        W2 = dequantize_nvfp4(weights["w2_codes"][e], weights["w2_scales"][e]).astype(dtype)
        y[o0:o1] = (Hq.astype(dtype) @ W2.T) * dtype(gh * np.float32(weights["w2_gscale"][e]))
    return y


def moe_layer_nvfp4(x, w_router, logit_bias, weights, k: int, I: int, x_gscale: float, h_gscale: float,
                    dtype=np.float32) -> dict:
    """O1..O8 with NVFP4 W4A4 experts."""
    E = w_router.shape[0]
    logits = router_logits(x, w_router, logit_bias)
    ids, gates = topk_softmax(logits, k)
    offsets, sorted_rows, row_pos, active = permute(ids, E)
    y_perm = expert_ffn_nvfp4(x, offsets, sorted_rows, k, weights, I, x_gscale, h_gscale, dtype=dtype)
    y = combine(y_perm, row_pos, gates)
    return dict(logits=logits, ids=ids, gates=gates, offsets=offsets, sorted_rows=sorted_rows,
                row_pos=row_pos, active=active, y_perm=y_perm, y=y)
