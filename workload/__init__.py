"""Seeded synthetic inputs for the routed-expert MoE layer with low-bit experts.

This module is the only code shared by the GPU path's callers (tests, bench) and
the CPU oracle.  It draws random numbers and stores them in the layer's input
formats; it performs none of the layer's arithmetic (no routing, no unpacking,
no dequantisation, no matmuls).

Input formats (all row-major, contiguous):

* ``x``          [T, H]        uint16 holding bfloat16 bits (round-to-nearest-even
                               from float32 samples).
* ``w_router``   [E, H]        uint16 bfloat16 bits.  The pages keep routers in
                               16-bit precision (page 1 "Qwen3.8-Flash-Next on one
                               24 GB GPU", opening paragraph; page 5 model card,
                               "Precision map").
* ``logit_bias`` [E] float32 or None: a log-prior added to router logits.
* ``w13_codes``  [E, 2I, H/P]  uint32 words, P = 32/bits codes per word, packed
                               along K (the reduction dimension), least
                               significant field first.  Rows [0, I) are the
                               gate projection, rows [I, 2I) the up projection.
* ``w13_scales`` [E, 2I, H/G] uint16 bfloat16 bits, one per G-wide K group
                               (G = 128, or 32 for the group-32 formats).
* ``w13_zeros``  [E, 2I, H/G]  uint8 zero-points (2-bit format only).
* ``w2_codes``   [E, H, I/P], ``w2_scales`` [E, H, I/G], ``w2_zeros`` likewise
                 for the down projection.

INT4 and 2-bit codes are drawn as uniformly random 32-bit words: every field
of a uniform word is uniform over its 2**bits values, so INT4 codes are
uniform over the 16 signed values and 2-bit codes uniform over {0..3}.  INT8
codes are drawn uniformly from -127..127 (the symmetric range, no -128) and
stored as the bytes q + 128, four per word, least significant first.  FP6
(bits = 6) rows are uniform random words, so every 6-bit e2m3 field is
uniform over the 64 codes; their scales are fp16 bits (|N(0,1)| * sigma,
rounded to nearest even), one per 128 K.

Each tensor gets its own PCG64 stream keyed by (workload seed, tensor tag,
weight-set index), so any one tensor can be regenerated alone.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

GROUP = 128  # quantisation group along K

# tensor tags for the per-tensor random streams
_TAG_X, _TAG_WR, _TAG_W13C, _TAG_W13S, _TAG_W13Z, _TAG_W2C, _TAG_W2S, _TAG_W2Z = range(8)


@dataclass(frozen=True)
class Spec:
    """Shape and sampling laws of one synthetic MoE-layer workload."""

    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    bits: int
    seed: int
    router_law: str = "normal"     # "normal": N(0, 0.02); "uniform": U(+-0.02*sqrt(3))
    zipf_s: float = 0.0            # >0: add -s*ln(e+1) to the logits of expert e
    x_law: str = "normal"          # "normal" or "ar1_streams"
    streams: int = 0               # ar1_streams: number of independent streams
    ar1_alpha: float = 0.85
    scale_sigma: float = 0.02      # scales are |N(0,1)| * scale_sigma
    group: int = 128               # quantisation group along K (128 or 32; 16 marks NVFP4)
    nv_gx: float = 2.0 ** -8       # NVFP4: tensor scales of the activation and h quantisers
    nv_gh: float = 2.0 ** -7
    nv_scale_codes: tuple = (0x28, 0x47)  # NVFP4: E4M3 group-scale codes drawn uniformly from this range
    n_sets: int = 1                # distinct weight sets cycled by the bench
    note: str = ""

    @property
    def words_per_row(self):
        """K -> packed uint32 words per row (FP6: 16 codes per 3 words)."""
        return lambda K: K * self.bits // 32

    def weight_bytes_per_expert(self) -> int:
        """Packed bytes one expert occupies: codes + bf16 scales (+ u8 zeros)."""
        H, I = self.H, self.I
        n_w = 2 * I * H + H * I                  # weights in gate_up and down
        codes = n_w * self.bits // 8
        groups = n_w // self.group
        if self.nvfp4:
            return codes + groups                # one E4M3 byte per group of 16
        zeros = groups if self.bits == 2 else 0
        return codes + 2 * groups + zeros

    @property
    def nvfp4(self) -> bool:
        return self.bits == 4 and self.group == 16


SPECS: Dict[str, Spec] = {
    s.name: s
    for s in [
        Spec("tiny_t4_h256_e8_k2_i128_int4", T=4, H=256, E=8, k=2, I=128, bits=4, seed=1000,
             note="CPU-seconds layer; N(0,0.02) router"),
        Spec("decode_t1_h4096_e256_k8_i1024_int4", T=1, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1001, router_law="uniform", n_sets=8,
             note="batch-1 decode; 8 weight sets cycled so touched bytes exceed the 256 MB Infinity Cache"),
        Spec("verify_t16_h4096_e256_k8_i1024_int4", T=16, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1002, router_law="uniform", x_law="ar1_streams", streams=4, n_sets=8,
             note="speculative verify: 4 streams x 4 draft tokens, AR(1) correlated activations"),
        Spec("prefill_t4096_h4096_e256_k8_i1024_int4", T=4096, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1003, zipf_s=1.1,
             note="prefill chunk; Zipf(1.1) log-prior on the router logits"),
        Spec("decode_t1_h4096_e256_k8_i1024_int2", T=1, H=4096, E=256, k=8, I=1024, bits=2,
             seed=1004, router_law="uniform", scale_sigma=0.05, n_sets=16,
             note="2-bit experts with zero-points, batch-1 decode, 16 sets cycled"),
        Spec("prefill_t8192_h4096_e256_k8_i1024_int2", T=8192, H=4096, E=256, k=8, I=1024, bits=2,
             seed=1005, zipf_s=1.1, scale_sigma=0.05,
             note="2-bit experts, prefill chunk with Zipf(1.1) log-prior"),
        Spec("decode_t1_h4096_e256_k8_i1024_int4g32", T=1, H=4096, E=256, k=8, I=1024, bits=4, group=32,
             seed=1007, router_law="uniform", n_sets=8,
             note="batch-1 decode, INT4 symmetric group-32 experts (the draft-layer format)"),
        Spec("decode_t1_h4096_e256_k8_i1024_int8", T=1, H=4096, E=256, k=8, I=1024, bits=8,
             seed=1008, router_law="uniform", scale_sigma=0.0015, n_sets=4,
             note="batch-1 decode, INT8 symmetric group-128 experts; 4 sets of 3.2 GB cycled"),
        Spec("decode_t1_h4096_e256_k8_i1024_int8g32", T=1, H=4096, E=256, k=8, I=1024, bits=8, group=32,
             seed=1009, router_law="uniform", scale_sigma=0.0015, n_sets=4,
             note="batch-1 decode, INT8 symmetric group-32 experts"),
        Spec("prefill_t4096_h4096_e256_k8_i1024_int8g32", T=4096, H=4096, E=256, k=8, I=1024, bits=8, group=32,
             seed=1010, zipf_s=1.1, scale_sigma=0.0015,
             note="prefill chunk, INT8 group-32 experts, Zipf(1.1) log-prior"),
        Spec("decode_t1_h4096_e256_k8_i1024_fp6", T=1, H=4096, E=256, k=8, I=1024, bits=6,
             seed=1011, router_law="uniform", n_sets=4,
             note="batch-1 decode, fp6 e2m3 experts with fp16 group-128 scales; 4 sets of 2.5 GB cycled"),
        Spec("prefill_t4096_h4096_e256_k8_i1024_fp6", T=4096, H=4096, E=256, k=8, I=1024, bits=6,
             seed=1012, zipf_s=1.1,
             note="prefill chunk, fp6 e2m3 experts, Zipf(1.1) log-prior"),
        Spec("decode_t1_h4096_e256_k8_i1024_nvfp4", T=1, H=4096, E=256, k=8, I=1024, bits=4, group=16,
             seed=1013, router_law="uniform", n_sets=8,
             note="batch-1 decode, NVFP4 W4A4 experts (E2M1, E4M3 scales per 16, tensor scales)"),
        Spec("prefill_t4096_h4096_e256_k8_i1024_nvfp4", T=4096, H=4096, E=256, k=8, I=1024, bits=4, group=16,
             seed=1014, zipf_s=1.1, note="prefill chunk, NVFP4 W4A4 experts, Zipf(1.1) log-prior"),
        Spec("mid_t64_h4096_e256_k8_i1024_int4", T=64, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1006, router_law="uniform", x_law="ar1_streams", streams=16, n_sets=2,
             note="middle batch: 16 streams x 4 draft tokens (higher-concurrency verify), decode path"),
        Spec("mid_t256_h4096_e256_k8_i1024_int4", T=256, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1015, router_law="uniform", x_law="ar1_streams", streams=64, n_sets=2,
             note="middle batch: 64 streams x 4 draft tokens, about 8 rows per expert"),
        Spec("mid_t512_h4096_e256_k8_i1024_int4", T=512, H=4096, E=256, k=8, I=1024, bits=4,
             seed=1016, router_law="uniform", x_law="ar1_streams", streams=128, n_sets=2,
             note="middle batch: 128 streams x 4 draft tokens, about 16 rows per expert"),
    ]
}


def spec(name: str, **overrides) -> Spec:
    """Look up a workload by name, optionally overriding fields (e.g. T, E, k)."""
    base = SPECS[name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return Spec(**d)


def _rng(seed: int, tag: int, set_idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, set_idx)))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def _uniform_words(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    n64 = (n + 1) // 2
    w = rng.bit_generator.random_raw(n64).view(np.uint32)[:n]
    return np.ascontiguousarray(w.reshape(shape))


def _int8_words(rng: np.random.Generator, shape) -> np.ndarray:
    """Words of four INT8 codes, each uniform over -127..127, stored as q + 128."""
    u = rng.integers(1, 256, size=tuple(shape[:-1]) + (4 * shape[-1],), dtype=np.uint8)
    return np.ascontiguousarray(u).view("<u4").astype(np.uint32)


def make_x(sp: Spec, set_idx: int = 0) -> np.ndarray:
    """Activations [T, H] as bf16 bits."""
    rng = _rng(sp.seed, _TAG_X, set_idx)
    if sp.x_law == "normal":
        xf = rng.standard_normal((sp.T, sp.H), dtype=np.float32)
    elif sp.x_law == "ar1_streams":
        # consecutive tokens of a stream: x_{j+1} = a*x_j + sqrt(1-a^2)*eps;
        # streams of ceil(T / streams) tokens fill the rows in order (T rows in all)
        n_streams = max(1, min(sp.streams, sp.T))
        per = -(-sp.T // n_streams)
        a = sp.ar1_alpha
        xf = np.empty((sp.T, sp.H), np.float32)
        for s in range(n_streams):
            cur = rng.standard_normal(sp.H, dtype=np.float32)
            for j in range(per):
                if s * per + j >= sp.T:
                    break
                if j:
                    eps = rng.standard_normal(sp.H, dtype=np.float32)
                    cur = (a * cur + math.sqrt(1.0 - a * a) * eps).astype(np.float32)
                xf[s * per + j] = cur
    else:
        raise ValueError(sp.x_law)
    return bf16_bits(xf)


def make_router(sp: Spec):
    """Router weight [E, H] (bf16 bits) and optional logit bias [E] (float32)."""
    rng = _rng(sp.seed, _TAG_WR)
    if sp.router_law == "normal":
        w = rng.standard_normal((sp.E, sp.H), dtype=np.float32) * np.float32(0.02)
    elif sp.router_law == "uniform":
        lim = 0.02 * math.sqrt(3.0)  # same standard deviation as N(0, 0.02)
        w = rng.uniform(-lim, lim, size=(sp.E, sp.H)).astype(np.float32)
    else:
        raise ValueError(sp.router_law)
    bias = None
    if sp.zipf_s > 0:
        rank = np.arange(1, sp.E + 1, dtype=np.float64)
        bias = (-sp.zipf_s * np.log(rank)).astype(np.float32)
    return bf16_bits(w), bias


def _scales(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    s = np.abs(rng.standard_normal(shape, dtype=np.float32)) * np.float32(sigma)
    return bf16_bits(s)


def _fp16_scales(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    s = np.abs(rng.standard_normal(shape, dtype=np.float32)) * np.float32(sigma)
    return s.astype(np.float16).view(np.uint16)


def _nvfp4_weight_set(sp: Spec, set_idx: int) -> Dict[str, np.ndarray]:
    """NVFP4 experts: E2M1 codes uniform over the 16 codes (uniform words, 8
    per word along K), E4M3 group scales drawn uniformly from the codes
    nv_scale_codes (by default 0x28..0x47, i.e. 0.25 .. 3.75; 0x01..0x7E spans
    every positive finite E4M3 value, subnormals and 448 included), float32
    tensor scales 0.004 * U(1, 1.25) per expert and projection."""
    E, H, I = sp.E, sp.H, sp.I
    out = {}
    for name, tc, ts, tz, (N, K) in (("w13", _TAG_W13C, _TAG_W13S, _TAG_W13Z, (2 * I, H)),
                                     ("w2", _TAG_W2C, _TAG_W2S, _TAG_W2Z, (H, I))):
        out[f"{name}_codes"] = _uniform_words(_rng(sp.seed, tc, set_idx), (E, N, K // 8))
        lo, hi = sp.nv_scale_codes
        out[f"{name}_scales"] = _rng(sp.seed, ts, set_idx).integers(lo, hi + 1, size=(E, N, K // 16), dtype=np.uint8)
        out[f"{name}_gscale"] = (0.004 * _rng(sp.seed, tz, set_idx).uniform(1.0, 1.25, size=E)).astype(np.float32)
    return out


def make_weight_set(sp: Spec, set_idx: int = 0) -> Dict[str, np.ndarray]:
    """One full layer of expert weights in the packed formats described above."""
    E, H, I, G = sp.E, sp.H, sp.I, sp.group
    nw = sp.words_per_row
    if sp.nvfp4:
        return _nvfp4_weight_set(sp, set_idx)
    if H % GROUP or I % GROUP:
        raise ValueError("H and I must be multiples of 128")
    if G not in (32, 128) or (G == 32 and sp.bits in (2, 6)):
        raise ValueError("group 128, or 32 for INT4 / INT8")
    codes = _int8_words if sp.bits == 8 else _uniform_words
    scales = _fp16_scales if sp.bits == 6 else _scales
    out = {
        "w13_codes": codes(_rng(sp.seed, _TAG_W13C, set_idx), (E, 2 * I, nw(H))),
        "w13_scales": scales(_rng(sp.seed, _TAG_W13S, set_idx), (E, 2 * I, H // G), sp.scale_sigma),
        "w2_codes": codes(_rng(sp.seed, _TAG_W2C, set_idx), (E, H, nw(I))),
        "w2_scales": scales(_rng(sp.seed, _TAG_W2S, set_idx), (E, H, I // G), sp.scale_sigma),
    }
    if sp.bits == 2:
        # integer zero-points drawn uniformly from {1, 2}
        out["w13_zeros"] = _rng(sp.seed, _TAG_W13Z, set_idx).integers(
            1, 3, size=(E, 2 * I, H // G), dtype=np.uint8)
        out["w2_zeros"] = _rng(sp.seed, _TAG_W2Z, set_idx).integers(
            1, 3, size=(E, H, I // G), dtype=np.uint8)
    return out


@dataclass
class LayerInputs:
    spec: Spec
    x: np.ndarray
    w_router: np.ndarray
    logit_bias: Optional[np.ndarray]
    weights: Dict[str, np.ndarray] = field(default_factory=dict)


def make_layer_inputs(name_or_spec, set_idx: int = 0, **overrides) -> LayerInputs:
    """Activations, router and one weight set of a workload."""
    sp = name_or_spec if isinstance(name_or_spec, Spec) else spec(name_or_spec, **overrides)
    w_r, bias = make_router(sp)
    return LayerInputs(sp, make_x(sp, set_idx), w_r, bias, make_weight_set(sp, set_idx))


def list_workloads() -> List[str]:
    return list(SPECS)
