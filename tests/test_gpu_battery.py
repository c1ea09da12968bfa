"""Kernel-level adversarial battery through both expert-FFN paths, every format.

Page "Qwen3.8-Flash-Next FP6-INT8", "Quantization quality", kernel level: the
pages check their GEMV and dequant kernels on every code in every group
position, under scale extremes and activation extremes.  Here the same is
done through the C ABI against the CPU oracle, for each weight format on the
decode path (T = 1 and T = 3) and on the grouped-GEMM path (T = 40):

* codes: at every K index k the rows n hold P_k[n mod C], P_k an independent
  random permutation of the format's C codes, so every code sits at every
  position of every group in both projections, while rows stay unrelated to
  one another (a plain walk (n + k) mod C would make each gate row equal its
  up row and every down row sum to zero, an output so ill-conditioned that
  rounding h to bf16 alone breaks a per-row bar);
* scales: a class per case, the whole matrix at one extreme (tiny, unit,
  large; for fp16 the subnormal 2^-24 range and the 65504 top; for E4M3 the
  subnormal codes and 448) or alternating extremes group by group;
* activations: tiny (2^-20), unit and large (2^8) normal samples, with
  exact zeros mixed in.

A second pass runs the full-chunk decode kernels (H = 4096, I = 1024: the
one-token per-group pipeline at T = 1, the row passes at T = 3) on the scale
classes.

Magnitudes are chosen so that every intermediate stays a normal float32 and
bf16 number.  Bars: y_perm and y within 2e-2 relative Frobenius error of the
float32 oracle, per row too (NVFP4: 99 % of rows, the rest within 5e-2, since
h is quantised from sums taken in different orders).
"""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_amd as bq
import oracle
import workload
from gpu_util import bf16_np_to_f32, row_rel_err, to_dev, to_np

pytestmark = pytest.mark.gpu
TOL = 2e-2
K_TOP = 2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------ inputs
def _pack(u, bits):
    """Fields u [..., K] (already offset, < 2^bits) -> words, least significant field first."""
    P = 32 // bits
    u = u.astype(np.uint32).reshape(u.shape[:-1] + (u.shape[-1] // P, P))
    w = np.zeros(u.shape[:-1], np.uint32)
    for i in range(P):
        w |= u[..., i] << np.uint32(bits * i)
    return w


def _pack_fp6(c):
    """6-bit codes [..., K] -> one little-endian bit stream per row (3 words per 16 codes)."""
    K = c.shape[-1]
    bitsarr = ((c[..., :, None].astype(np.uint64) >> np.arange(6, dtype=np.uint64)) & np.uint64(1)).astype(np.uint8)
    stream = bitsarr.reshape(c.shape[:-1] + (6 * K,))
    b32 = stream.reshape(c.shape[:-1] + (6 * K // 32, 32)).astype(np.uint64)
    return (b32 << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)


def _cover(N, K, C, rng):
    """[N, K] codes: column k is P_k[n mod C] for a random permutation P_k of 0..C-1."""
    P = np.argsort(rng.random((K, C)), axis=1)                   # K independent permutations
    return P[np.arange(K)[None, :], (np.arange(N) % C)[:, None]]


# format id -> (bits, group, number of codes)
FORMATS = {"int4_g128": (4, 128), "int4_g32": (4, 32), "int2_g128": (2, 128), "int8_g128": (8, 128),
           "int8_g32": (8, 32), "fp6_g128": (6, 128), "nvfp4": (4, 16)}

# scale classes: a function of (rng, shape) -> scale values (float), per format family
def _bf16_scales(cls, rng, shape):
    u = 1.0 + rng.random(shape)
    if cls == "tiny":
        v = u * 2.0 ** -30
    elif cls == "unit":
        v = u
    elif cls == "large":
        v = u * 2.0 ** 12
    else:  # alternating extremes along K groups
        g = np.arange(shape[-1]) % 2
        v = u * np.where(g == 0, 2.0 ** -30, 2.0 ** 12)
    return workload.bf16_bits(v.astype(np.float32))


def _fp16_scales(cls, rng, shape):
    if cls == "tiny":          # fp16 subnormals: m * 2^-24, m = 1..7
        v = rng.integers(1, 8, shape) * 2.0 ** -24
    elif cls == "unit":
        v = 1.0 + rng.random(shape)
    elif cls == "large":       # up to the fp16 maximum 65504
        v = np.minimum(2.0 ** 15 * (1.0 + rng.random(shape)), 65504.0)
    else:
        g = np.arange(shape[-1]) % 2
        v = np.where(g == 0, rng.integers(1, 8, shape) * 2.0 ** -24, 65504.0)
    return v.astype(np.float16).view(np.uint16)


def _e4m3_codes(cls, rng, shape):
    if cls == "tiny":          # subnormal E4M3: 2^-9 .. 7 * 2^-9
        c = rng.integers(0x01, 0x08, shape)
    elif cls == "unit":
        c = rng.integers(0x30, 0x41, shape)
    elif cls == "large":       # the top binade, up to 448
        c = rng.integers(0x78, 0x7F, shape)
    else:
        g = np.arange(shape[-1]) % 2
        c = np.where(g == 0, rng.integers(0x01, 0x08, shape), rng.integers(0x78, 0x7F, shape))
    return c.astype(np.uint8)


def _weights(fmt, cls, seed, H, I, E):
    bits, group = FORMATS[fmt]
    rng = np.random.default_rng(seed)
    out = {}
    for name, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
        if fmt == "nvfp4":
            out[f"{name}_codes"] = np.stack([_pack(_cover(N, K, 16, rng), 4) for _ in range(E)])
            out[f"{name}_scales"] = _e4m3_codes(cls, rng, (E, N, K // 16))
            out[f"{name}_gscale"] = (2.0 ** -6 * (1.0 + rng.random(E))).astype(np.float32)
            continue
        if bits == 6:
            out[f"{name}_codes"] = np.stack([_pack_fp6(_cover(N, K, 64, rng)) for _ in range(E)])
            sc = _fp16_scales(cls, rng, (E, N, K // group))
        else:
            C = {4: 16, 2: 4, 8: 255}[bits]
            off = 1 if bits == 8 else 0                            # INT8 fields 1..255 (q = -127..127)
            out[f"{name}_codes"] = np.stack([_pack(_cover(N, K, C, rng) + off, bits) for _ in range(E)])
            sc = _bf16_scales(cls, rng, (E, N, K // group))
        out[f"{name}_scales"] = sc
        if bits == 2:
            out[f"{name}_zeros"] = (1 + (np.arange(K // group)[None, None, :] + np.arange(N)[None, :, None]
                                         + np.arange(E)[:, None, None]) % 2).astype(np.uint8)
    return out


def _x(T, act, seed, H):
    rng = np.random.default_rng(seed)
    mag = {"tiny": 2.0 ** -20, "unit": 1.0, "large": 2.0 ** 8}[act]
    x = rng.standard_normal((T, H)) * mag
    x[rng.random((T, H)) < 0.05] = 0.0
    return workload.bf16_bits(x.astype(np.float32)), mag


def _dev_weights(w):
    return {kk: to_dev(v) for kk, v in w.items()}


def _nvfp4_h_gscale(x, wts, off, srt, gx, I):
    """A tensor scale for h that puts the largest |h| of the case at 64 times
    6 * gh, inside the E4M3 x E2M1 range (h computed on the CPU with the
    oracle's quantiser and dequantiser, as its FFN does)."""
    xf = oracle.bf16_to_f32(x)
    hmax = 0.0
    for e in range(off.size - 1):
        if off[e + 1] == off[e]:
            continue
        _, xq = oracle.quant_nvfp4(xf[srt[off[e]:off[e + 1]] // K_TOP], gx)
        W13 = oracle.dequantize_nvfp4(wts["w13_codes"][e], wts["w13_scales"][e])
        A = (xq @ W13.T) * np.float32(gx * wts["w13_gscale"][e])
        hmax = max(hmax, float(np.abs(oracle.silu(A[:, :I]) * A[:, I:]).max()))
    return hmax / (6.0 * 64.0) if hmax > 0 else 1.0


# ------------------------------------------------------------------ the battery
CASES = [(s, a) for s in ("tiny", "unit", "large", "mixed") for a in ("tiny", "unit", "large")]
FULL_CASES = [("tiny", "unit"), ("unit", "unit"), ("large", "unit"), ("mixed", "unit"), ("unit", "tiny"),
              ("large", "large")]


def _run(fmt, T, H, I, E, cases, seed0):
    bits, group = FORMATS[fmt]
    nv = fmt == "nvfp4"
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=K_TOP, seed=seed0 + T)
    w_r, _ = workload.make_router(sp)
    ws = bq.Workspaces("cuda")
    say(f"[gpu-test] battery {fmt} T={T} H={H} I={I}: {len(cases)} scale x activation cases")
    worst = 0.0
    for ci, (scls, acls) in enumerate(cases):
        wts = _weights(fmt, scls, 100 * ci + T, H, I, E)
        x, mag = _x(T, acls, 200 * ci + T, H)
        xd = to_dev(x)
        r = bq.route_permute(xd, to_dev(w_r), K_TOP, ws=ws)
        off, srt, rp = to_np(r["offsets"]), to_np(r["sorted_rows"]), to_np(r["row_pos"])
        g = to_np(r["gates"])
        wd = _dev_weights(wts)
        if nv:
            gx = mag * 2.0 ** -8
            gh = _nvfp4_h_gscale(x, wts, off, srt, gx, I)
            yp = bq.expert_ffn_nvfp4(xd, r["offsets"], r["sorted_rows"], r["active"], K_TOP, wd, I, gx, gh, ws=ws)
            ref = oracle.expert_ffn_nvfp4(x, off, srt, K_TOP, wts, I, gx, gh)
        else:
            yp = bq.expert_ffn(xd, r["offsets"], r["sorted_rows"], r["active"], K_TOP, wd, bits, I, ws=ws,
                               group=group)
            ref = oracle.expert_ffn(x, off, srt, K_TOP, wts, bits, I, group=group)
        y = bq.combine(yp, r["row_pos"], r["gates"])
        ypf, yf = bf16_np_to_f32(to_np(yp)), bf16_np_to_f32(to_np(y))
        assert np.all(np.isfinite(ref)) and np.all(np.isfinite(ypf)), (scls, acls)
        yref = oracle.combine(ref, rp, g)
        e1, e2 = oracle.rel_fro(ypf, ref), oracle.rel_fro(yf, yref)
        rows = row_rel_err(ypf, ref)
        worst = max(worst, e1, e2)
        msg = f"{fmt} T={T} scales {scls}, x {acls}: y_perm {e1:.2e}, y {e2:.2e}, worst row {rows.max():.2e}"
        assert e1 <= TOL and e2 <= TOL, msg
        if nv:
            assert (rows <= TOL).mean() >= 0.99 and rows.max() <= 5e-2, msg
        else:
            assert rows.max() <= TOL, msg
        del wd
    say(f"    worst rel-fro over the cases {worst:.2e}")
    ws.check()


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("T", [1, 3, 40], ids=lambda t: f"T{t}")
def test_ffn_battery(fmt, T):
    """H = 256, I = 128, E = 4, top-2: decode path at T = 1, 3, grouped GEMM at T = 40."""
    _run(fmt, T, 256, 128, 4, CASES, 7000)


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("T", [1, 3], ids=lambda t: f"T{t}")
def test_ffn_battery_full_chunks(fmt, T):
    """H = 4096, I = 1024, E = 2, top-2: the full-chunk decode kernels."""
    _run(fmt, T, 4096, 1024, 2, FULL_CASES, 7100)
