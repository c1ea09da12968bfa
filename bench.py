#!/usr/bin/env python3
"""Throughput of the routed-expert MoE layer with low-bit experts on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager] [--no-cpu-baseline]
                    [--no-configs] [--no-peaks] [--experts arrays|table|host] [--stages]
    python bench.py --peaks-only          # the device's measured stream-read and MFMA rates
    python bench.py --copy-calibration    # a plain copy of known size, to scale HBM traffic counters

A step is one pass of the whole layer over one batch of synthetic input
already resident in HBM, through the C ABI: for T <= 4 one moe_layer_w4a16 /
_w2a16 call (router, grouping, expert FFN and combine in one launch; --stages
runs the stage calls instead), for larger T moe_route_permute,
moe_expert_ffn_w4a16/_w2a16 and moe_combine.  Decode workloads cycle through
their distinct weight sets (and activations) step by step, so the expert bytes
a step touches come from HBM rather than the 256 MB Infinity Cache.  Each
step is replayed from a HIP graph holding one step per weight set (--eager
launches the calls one by one instead).

The default run times the headline workload (decode T = 1, INT4 group 128:
exactly --steps steps after --warmup) and then the other four configurations
of the layer (verify T = 16 INT4, prefill T = 4096 INT4, 2-bit decode T = 1,
2-bit prefill T = 8192) under "configs", each with at least 100 (decode) or
20 (prefill) timed steps.  For every workload it reports tokens/s, the step
time's median / p10 / p90 over back-to-back graph replays, the roofline of
the dominant kernel (decode and middle batches: HBM-bound on the packed
weight bytes of the selected experts; prefill: the expert-FFN GEMMs,
MFMA-bound on useful FLOPs)
timed with HIP events on the stream it is launched on, that rate also as a
fraction of the rates this device measurably reaches (a streaming read and an
MFMA-only loop, "peaks"), and the CPU oracle's rate on a bounded sample of
the same workload, timed on the host in child processes pinned to distinct
cores.  --experts table / host run the expert FFN through the address-table
entry points with the experts in HBM / in pinned host memory read over PCIe.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; decode HBM GB/s % peak; prefill MFMA % peak (1 GPU)"
DEFAULT_WORKLOAD = "decode_t1_h4096_e256_k8_i1024_int4"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
PCIE_PEAK_GBS = 63.0  # PCIe 5.0 x16, one direction: 16 lanes x 32 GT/s x 128/130 / 8
FUSED_MAX_T = 8  # batches up to this size run as one moe_layer launch (measured faster up to 8 tokens); larger ones as the stages


CONFIGS = [  # the layer's other configurations, timed after the headline one
    ("verify_t16_h4096_e256_k8_i1024_int4", "decode verify T=16 (4 streams x 4 drafts), INT4 g128"),
    ("prefill_t4096_h4096_e256_k8_i1024_int4", "prefill T=4096, INT4 g128, Zipf(1.1) routing"),
    ("decode_t1_h4096_e256_k8_i1024_int2", "decode T=1, 2-bit g128 with zero-points"),
    ("prefill_t8192_h4096_e256_k8_i1024_int2", "prefill T=8192, 2-bit g128, Zipf(1.1) routing"),
]
MIN_STEPS_DECODE, MIN_STEPS_PREFILL = 100, 20


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, help="time this workload alone (default: the headline + configs)")
    ap.add_argument("--eager", action="store_true", help="launch the four calls per step without a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-peaks", action="store_true", help="skip the stream-read and MFMA-loop probes")
    ap.add_argument("--peaks-only", action="store_true", help="only run the stream-read and MFMA-loop probes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--ffn-only", action="store_true", help="time only the expert-FFN stage launches (for profiling)")
    ap.add_argument("--stages", action="store_true", help="decode: run the stage calls instead of the one-launch layer")
    ap.add_argument("--experts", choices=("arrays", "table", "host"), default="arrays",
                    help="expert weights as stacked arrays, through an address table (HBM), or in pinned host memory")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


COPY_BYTES = 256 << 20


def copy_calibration():
    """Four device-to-device copies of COPY_BYTES each (reads and writes COPY_BYTES per launch)."""
    import torch

    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": 4}), flush=True)


# Sources of each dominant kernel: a stored traffic figure is reported only
# while these files are unchanged since the counters were taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "decode": ["bit_quantized_moe_amd/csrc/ffn_decode.hip", "bit_quantized_moe_amd/csrc/gemv_ops.cuh",
               "bit_quantized_moe_amd/csrc/common.cuh", "bit_quantized_moe_amd/csrc/route_dev.cuh"],
    "layer": ["bit_quantized_moe_amd/csrc/ffn_decode.hip", "bit_quantized_moe_amd/csrc/gemv_ops.cuh",
              "bit_quantized_moe_amd/csrc/common.cuh", "bit_quantized_moe_amd/csrc/route_dev.cuh"],
    "mid": ["bit_quantized_moe_amd/csrc/ffn_mid.hip", "bit_quantized_moe_amd/csrc/gemv_ops.cuh",
            "bit_quantized_moe_amd/csrc/common.cuh"],
    "prefill": ["bit_quantized_moe_amd/csrc/ffn_prefill.hip", "bit_quantized_moe_amd/csrc/ffn_mid.hip",
                "bit_quantized_moe_amd/csrc/gemv_ops.cuh", "bit_quantized_moe_amd/csrc/common.cuh"],
}


def sources_digest(kind):
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload, kind):
    """HBM bytes per launch measured with FETCH_SIZE / WRITE_SIZE (scaled by a plain copy), or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload if kind != "layer" else workload + ":layer")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != sources_digest(kind):
        return None
    return int(rec["hbm_bytes_per_launch"])


def start_cpu_baseline(args, name, slot):
    """The oracle's rate on a bounded sample of `name`, in a child process pinned to its own core."""
    if args.no_cpu_baseline:
        return None
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    cores = sorted(os.sched_getaffinity(0))
    core = cores[-1 - slot % len(cores)]
    cmd = [sys.executable, "-m", "oracle.cpu_baseline", "--workload", name, "--seconds", str(args.cpu_seconds),
           "--core", str(cores.index(core))]
    return subprocess.Popen(cmd, cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def finish_cpu_baseline(proc):
    if proc is None:
        return None
    out, err = proc.communicate(timeout=900)
    if proc.returncode != 0:
        print(f"[bench] cpu baseline failed: {err[-500:]}", file=sys.stderr, flush=True)
        return None
    d = json.loads(out.strip().splitlines()[-1])
    return {k: d[k] for k in ("value", "unit", "cores", "kind", "sample", "host_cpus")}


class Plan:
    """Device buffers and pre-bound C-ABI calls for one workload."""

    def __init__(self, sp, dev, fused=False, experts="arrays"):
        import numpy as np
        import torch

        import bit_quantized_moe_amd as bq
        import workload

        self.sp, self.dev, self.L = sp, dev, bq.lib()
        self.fused = fused
        self.experts = experts
        T, H, E, k, I = sp.T, sp.H, sp.E, sp.k, sp.I
        n = T * k

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            if a.dtype == np.uint32:
                return torch.from_numpy(a.view(np.int32)).to(dev)
            return torch.from_numpy(a).to(dev)

        w_r, bias = workload.make_router(sp)
        self.w_r = up(w_r)
        self.bias = up(bias) if bias is not None else None
        self.sets = []
        t0 = time.time()
        # host memory is not cached by the GPU, so two sets are enough there
        self.n_sets = min(sp.n_sets, 2) if experts == "host" else sp.n_sets
        for s in range(self.n_sets):
            w = workload.make_weight_set(sp, s)
            if experts == "host":   # every expert's blocks in pinned host memory
                as_torch = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16}
                dw = {kk: torch.from_numpy(np.ascontiguousarray(v).view(as_torch.get(v.dtype, v.dtype))).pin_memory()
                      for kk, v in w.items()}
            else:
                dw = {kk: up(v) for kk, v in w.items()}
            del w
            st = dict(w=dw, x=up(workload.make_x(sp, s)))
            if experts != "arrays":
                st["table"] = bq.expert_table(dw, sp.bits, device=dev)
            st["ids"] = torch.empty((T, k), dtype=torch.int32, device=dev)
            st["gates"] = torch.empty((T, k), dtype=torch.float32, device=dev)
            st["offsets"] = torch.empty(E + 1, dtype=torch.int32, device=dev)
            st["sorted_rows"] = torch.empty(n, dtype=torch.int32, device=dev)
            st["row_pos"] = torch.empty(n, dtype=torch.int32, device=dev)
            st["active"] = torch.empty(1 + min(E, n), dtype=torch.int32, device=dev)
            self.sets.append(st)
        print(f"[bench] {self.n_sets} weight set(s) generated and uploaded in {time.time() - t0:.1f} s", flush=True)
        self.y_perm = torch.empty((n, H), dtype=torch.bfloat16, device=dev)
        self.y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.ws_route = torch.zeros(self.L.moe_route_permute_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
        ffn_ws = (self.L.moe_expert_ffn_nvfp4_workspace_size if sp.nvfp4 else self.L.moe_expert_ffn_workspace_size)
        self.ws_ffn = torch.zeros(ffn_ws(T, k, E, H, I), dtype=torch.uint8, device=dev)
        self.ws_layer = (torch.zeros(self.L.moe_layer_workspace_size(T, k, E, H, I), dtype=torch.uint8, device=dev)
                         if fused else None)
        self.torch = torch

    def _chk(self, s, name):
        if s != 0:
            raise RuntimeError(f"{name}: status {s}: {self.L.moe_last_error().decode()}")

    def route_permute(self, i):
        sp, st, L = self.sp, self.sets[i], self.L
        stream = self.torch.cuda.current_stream(self.dev).cuda_stream
        self._chk(L.moe_route_permute(st["x"].data_ptr(), self.w_r.data_ptr(),
                                      self.bias.data_ptr() if self.bias is not None else None, sp.T, sp.H, sp.E, sp.k,
                                      st["ids"].data_ptr(), st["gates"].data_ptr(), None, st["offsets"].data_ptr(),
                                      st["sorted_rows"].data_ptr(), st["row_pos"].data_ptr(), st["active"].data_ptr(),
                                      self.ws_route.data_ptr(), self.ws_route.numel(), stream), "moe_route_permute")

    def ffn(self, i):
        sp, st, L = self.sp, self.sets[i], self.L
        stream = self.torch.cuda.current_stream(self.dev).cuda_stream
        w = st["w"]
        common = (st["x"].data_ptr(), st["offsets"].data_ptr(), st["sorted_rows"].data_ptr(), st["active"].data_ptr(),
                  sp.T, sp.k, sp.E, sp.H, sp.I)
        if sp.nvfp4:
            s = L.moe_expert_ffn_nvfp4(*common, sp.nv_gx, sp.nv_gh, w["w13_codes"].data_ptr(),
                                       w["w13_scales"].data_ptr(), w["w13_gscale"].data_ptr(), w["w2_codes"].data_ptr(),
                                       w["w2_scales"].data_ptr(), w["w2_gscale"].data_ptr(), self.y_perm.data_ptr(),
                                       self.ws_ffn.data_ptr(), self.ws_ffn.numel(), stream)
        elif self.experts != "arrays":
            fn = L.moe_expert_ffn_w4a16_table if sp.bits == 4 else L.moe_expert_ffn_w2a16_table
            s = fn(*common, st["table"].data_ptr(), self.y_perm.data_ptr(), self.ws_ffn.data_ptr(),
                   self.ws_ffn.numel(), stream)
        elif sp.bits not in (2, 4) or sp.group != 128:
            s = L.moe_expert_ffn_wna16(*common, sp.bits, sp.group, w["w13_codes"].data_ptr(),
                                       w["w13_scales"].data_ptr(), None, w["w2_codes"].data_ptr(),
                                       w["w2_scales"].data_ptr(), None, self.y_perm.data_ptr(),
                                       self.ws_ffn.data_ptr(), self.ws_ffn.numel(), stream)
        elif sp.bits == 4:
            s = L.moe_expert_ffn_w4a16(*common, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                       w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(), self.y_perm.data_ptr(),
                                       self.ws_ffn.data_ptr(), self.ws_ffn.numel(), stream)
        else:
            s = L.moe_expert_ffn_w2a16(*common, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                       w["w13_zeros"].data_ptr(), w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(),
                                       w["w2_zeros"].data_ptr(), self.y_perm.data_ptr(), self.ws_ffn.data_ptr(),
                                       self.ws_ffn.numel(), stream)
        self._chk(s, "moe_expert_ffn")

    def combine(self, i):
        sp, st = self.sp, self.sets[i]
        stream = self.torch.cuda.current_stream(self.dev).cuda_stream
        self._chk(self.L.moe_combine(self.y_perm.data_ptr(), st["row_pos"].data_ptr(), st["gates"].data_ptr(), sp.T,
                                     sp.k, sp.H, self.y.data_ptr(), stream), "moe_combine")

    def layer(self, i):
        sp, st, L = self.sp, self.sets[i], self.L
        stream = self.torch.cuda.current_stream(self.dev).cuda_stream
        w = st["w"]
        head = (st["x"].data_ptr(), self.w_r.data_ptr(), self.bias.data_ptr() if self.bias is not None else None,
                sp.T, sp.H, sp.E, sp.k, sp.I)
        tail = (self.y.data_ptr(), st["ids"].data_ptr(), st["gates"].data_ptr(), self.ws_layer.data_ptr(),
                self.ws_layer.numel(), stream)
        if sp.nvfp4:
            s = L.moe_layer_nvfp4(*head[:8], sp.nv_gx, sp.nv_gh, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                  w["w13_gscale"].data_ptr(), w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(),
                                  w["w2_gscale"].data_ptr(), *tail)
        elif sp.bits not in (2, 4) or sp.group != 128:
            s = L.moe_layer_wna16(*head, sp.bits, sp.group, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                  None, w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(), None, *tail)
        elif sp.bits == 4:
            s = L.moe_layer_w4a16(*head, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                  w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(), *tail)
        else:
            s = L.moe_layer_w2a16(*head, w["w13_codes"].data_ptr(), w["w13_scales"].data_ptr(),
                                  w["w13_zeros"].data_ptr(), w["w2_codes"].data_ptr(), w["w2_scales"].data_ptr(),
                                  w["w2_zeros"].data_ptr(), *tail)
        self._chk(s, "moe_layer")

    def stages(self, i):
        self.route_permute(i)
        self.ffn(i)
        self.combine(i)

    def step(self, i):
        if self.fused:
            self.layer(i)
        else:
            self.stages(i)


def host_copy_rate(torch, dev):
    """GB/s of a plain pinned-host to device copy of 256 MiB (the link as torch drives it)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8).pin_memory()
    dst = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    b.record()
    torch.cuda.synchronize(dev)
    return 4 * COPY_BYTES / (a.elapsed_time(b) * 1e-3) / 1e9


def _pct(vals):
    import numpy as np

    v = np.asarray(vals, dtype=np.float64)
    return {"median": round(float(np.median(v)), 5), "p10": round(float(np.percentile(v, 10)), 5),
            "p90": round(float(np.percentile(v, 90)), 5)}


def measure_peaks(dev):
    """The device's measured rates: a streaming read of 1 GiB, streaming reads of 52 MB (the decode
    step's packed bytes, cycled over eight buffers so that no read hits the Infinity Cache), and an
    MFMA-only loop (bf16 16x16x32)."""
    import torch

    import bit_quantized_moe_amd as bq

    L = bq.lib()
    stream = torch.cuda.Stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(L.moe_probe_stream_blocks(1 << 30), dtype=torch.int32, device=dev)
    res = {}
    with torch.cuda.stream(stream):
        st = stream.cuda_stream

        def timed(fn, reps):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            fn(0)
            torch.cuda.synchronize(dev)
            ev[0].record(stream)
            for i in range(reps):
                fn(i)
                ev[i + 1].record(stream)
            torch.cuda.synchronize(dev)
            return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]

        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)

        def rd_big(i):
            if L.moe_probe_stream_read(big.data_ptr(), big.numel(), out.data_ptr(), st):
                raise RuntimeError(L.moe_last_error().decode())
        t = timed(rd_big, 20)
        res["hbm_stream_read_1GiB_GBs"] = round(big.numel() / (min(t) * 1e-3) / 1e9, 1)
        res["hbm_stream_read_1GiB_GBs_median"] = round(big.numel() / (sorted(t)[len(t) // 2] * 1e-3) / 1e9, 1)
        del big
        nb = 51904512
        chunks = [torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1) for _ in range(8)]

        def rd_small(i):
            c = chunks[i % 8]
            if L.moe_probe_stream_read(c.data_ptr(), c.numel(), out.data_ptr(), st):
                raise RuntimeError(L.moe_last_error().decode())
        t = timed(rd_small, 80)
        med = sorted(t)[len(t) // 2]
        res["hbm_stream_read_52MB_GBs"] = round(nb / (med * 1e-3) / 1e9, 1)
        res["hbm_stream_read_52MB_us"] = round(med * 1e3, 2)

        # the same reads eight in a row between two events, as the decode graphs run their steps
        def rd_eight(i):
            for j in range(8):
                rd_small(8 * i + j)
        t = timed(rd_eight, 20)
        med = sorted(t)[len(t) // 2] / 8
        res["hbm_stream_read_52MB_b2b_GBs"] = round(nb / (med * 1e-3) / 1e9, 1)
        res["hbm_stream_read_52MB_b2b_us"] = round(med * 1e3, 2)
        del chunks
        mblocks, iters = 2 * cus, 20000
        fout = torch.empty(4 * mblocks, dtype=torch.float32, device=dev)

        def mf(i):
            if L.moe_probe_mfma(mblocks, iters, fout.data_ptr(), st):
                raise RuntimeError(L.moe_last_error().decode())
        t = timed(mf, 10)
        flops = mblocks * 4 * iters * 8 * 16384.0
        res["mfma_bf16_TFLOPs"] = round(flops / (sorted(t)[len(t) // 2] * 1e-3) / 1e12, 1)
    res["probes"] = ("moe_probe_stream_read over 1 GiB (best of 20) and over 52 MB buffers cycled eight-fold "
                     "(median of 80 single launches; b2b: median of 20 groups of eight launches between two events, "
                     "per launch), eight 16-byte loads in flight per thread; moe_probe_mfma, "
                     f"{2 * cus} blocks of four waves, v_mfma_f32_16x16x32_bf16 on register operands, eight "
                     "independent accumulators (median of 10)")
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    return res


def run_workload(name, args, dev, steps, warmup):
    """Times one workload; returns the dict of its JSON entry."""
    import torch

    import bit_quantized_moe_amd as bq
    import workload

    sp = workload.spec(name)
    # the one-launch layer takes every format from stacked arrays
    fused = sp.T <= FUSED_MAX_T and not args.stages and args.experts == "arrays"
    plan = Plan(sp, dev, fused=fused, experts=args.experts)
    nset = plan.n_sets
    stream = torch.cuda.Stream(dev)

    def time_graph(fn):
        """Average time of fn(i) (one launch) over back-to-back replays of a graph of all sets."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(nset):
                fn(i)
        reps = max(1, max(steps, 40) // nset)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / (reps * nset)

    use_graph = not args.eager
    with torch.cuda.stream(stream):
        for i in range(nset):      # eager warm-up; fills every set's routing buffers (the FFN stage reads them)
            plan.stages(i)
            if fused:
                plan.layer(i)
        torch.cuda.synchronize(dev)

        # Steps run back to back as in a model's forward pass: one graph holds
        # one step per weight set (set i on step i), and single-step graphs
        # make up a remainder, so exactly K steps are timed.
        graphs = []
        g_all = None
        if use_graph:
            for i in range(nset):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    plan.step(i)
                graphs.append(g)
            g_all = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_all, stream=stream):
                for i in range(nset):
                    plan.step(i)
            torch.cuda.synchronize(dev)

        def run_steps(n):
            if use_graph:
                for _ in range(n // nset):
                    g_all.replay()
                for i in range(n % nset):
                    graphs[i].replay()
            else:
                for i in range(n):
                    plan.step(i % nset)

        # ---- whole-layer steps: exactly `steps` timed after `warmup`
        run_steps(warmup)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0 = time.perf_counter()
        e0.record(stream)
        if not args.ffn_only:
            run_steps(steps)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - c0
        ms_step = e0.elapsed_time(e1) / max(1, steps)

        # ---- step-time distribution: back-to-back replays of the graph of all sets, one event between
        # replays; each sample is one replay's time per step
        reps = max(10, -(-max(steps, MIN_STEPS_DECODE if sp.T <= 512 else MIN_STEPS_PREFILL) // nset))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for r in range(reps):
            if use_graph:
                g_all.replay()
            else:
                for i in range(nset):
                    plan.step(i)
            ev[r + 1].record(stream)
        torch.cuda.synchronize(dev)
        dist = _pct([ev[r].elapsed_time(ev[r + 1]) / nset for r in range(reps)])
        dist["samples"] = f"{reps} back-to-back replays of {nset} step(s), time per step of each"

        # ---- the expert-FFN stage alone, and (decode) the one-launch layer kernel alone
        ffn_ms = time_graph(plan.ffn)
        layer_ms = time_graph(plan.layer) if fused and not args.ffn_only else None

    flags = 0
    for buf in (plan.ws_route, plan.ws_ffn, plan.ws_layer):
        if buf is not None:
            flags |= bq.workspace_status(buf)
    if flags:
        raise RuntimeError(f"{name}: a bounded wait timed out during the run: the timings are not valid")

    # distinct experts per launch (decode bytes) from each set's routing
    distinct = [int(st["active"][0].item()) for st in plan.sets]
    mean_distinct = sum(distinct) / len(distinct)
    bpe = sp.weight_bytes_per_expert()
    # the library's expert-FFN dispatch: the decode and mid paths stream each
    # active expert's packed weights (HBM-bound), the grouped GEMMs are MFMA-bound
    path = bq.ffn_path(sp.T, sp.k, sp.E, sp.H, sp.I, "nvfp4" if sp.nvfp4 else sp.bits, sp.group)
    decode = path in ("decode", "mid")
    ffn_kernel = ("quant_nvfp4_kernel, then " if sp.nvfp4 else "") + {
        "decode": f"ffn_decode_kernel<{5 if sp.nvfp4 else sp.bits}, ...> (expert-FFN stage: gate_up+SwiGLU+down GEMV)",
        "mid": f"mid_kernel<{sp.bits}, true> gate_up+SwiGLU, then mid_kernel<{sp.bits}, false> down "
               "(rows staged per K step, each expert's weights streamed once per 32 rows)",
        "gemm": ("mid_kernel (experts of at most 64 rows), " if not sp.nvfp4 and sp.group == 128 and sp.bits in (2, 4)
                 else "") + "ffn_gemm_kernel gate_up+SwiGLU, then ffn_gemm_kernel down (grouped bf16-MFMA GEMMs)"}[path]
    ffn_stage = None
    if path == "decode" and args.experts == "host":
        alg = mean_distinct * bpe
        achieved = alg / (ffn_ms * 1e-3) / 1e9
        roof = {"bound": "pcie", "achieved": round(achieved, 1), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PCIE_PEAK_GBS, 4), "traffic": None,
                "kernel": "ffn_decode_kernel (address table, experts read in place from pinned host memory)",
                "algorithmic_bytes_per_launch": int(alg), "avg_launch_us": round(ffn_ms * 1e3, 3),
                "distinct_experts_per_launch": mean_distinct,
                "host_to_device_copy_GBs": round(host_copy_rate(torch, dev), 1)}
    elif decode:
        alg = mean_distinct * bpe
        achieved = alg / (ffn_ms * 1e-3) / 1e9
        ffn_stage = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(sp.name, path) if args.experts == "arrays" else None,
                     "kernel": ffn_kernel, "algorithmic_bytes_per_launch": int(alg),
                     "avg_launch_us": round(ffn_ms * 1e3, 3), "distinct_experts_per_launch": mean_distinct}
        roof = ffn_stage
        if layer_ms is not None:
            alg_l = alg + sp.E * sp.H * 2          # plus the bf16 router weights
            ach_l = alg_l / (layer_ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach_l, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach_l / HBM_PEAK_GBS, 4), "traffic": stored_traffic(sp.name, "layer"),
                    "kernel": "ffn_decode_kernel LAYER (one launch: router, top-k, grouping, expert FFN, combine)",
                    "algorithmic_bytes_per_launch": int(alg_l), "avg_launch_us": round(layer_ms * 1e3, 3),
                    "distinct_experts_per_launch": mean_distinct}
    else:
        flops = 2.0 * sp.T * sp.k * 3 * sp.H * sp.I
        achieved = flops / (ffn_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": stored_traffic(sp.name, "prefill") if args.experts == "arrays" else None,
                "kernel": "expert FFN call (" + ffn_kernel + ")",
                "algorithmic_flops_per_launch": flops, "avg_launch_us": round(ffn_ms * 1e3, 3)}
    tok_s = sp.T / (ms_step * 1e-3) if ms_step > 0 else 0.0
    entry = {
        "value": round(tok_s, 1), "unit": "tokens/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5), "step_ms": dist,
        "config": {"workload": sp.name, "T": sp.T, "H": sp.H, "E": sp.E, "top_k": sp.k, "I": sp.I,
                   "weight_format": ("nvfp4 w4a4 (e2m1, e4m3 scales per 16)" if sp.nvfp4 else
                                     "fp6 e2m3 g128 (fp16 scales)" if sp.bits == 6 else
                                     f"int{sp.bits} g{sp.group}" + (" + zero-point" if sp.bits == 2 else " sym")),
                   "weight_sets_cycled": nset, "experts": args.experts,
                   "launch": f"hip graph of {nset} steps (one per weight set)" if use_graph else "eager",
                   "step": "moe_layer (one launch)" if fused else "stage calls",
                   "wall_s_timed": round(wall, 4)},
        "roofline": roof,
    }
    if ffn_stage is not None and layer_ms is not None:
        entry["ffn_stage"] = ffn_stage
    del plan, graphs, g_all
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    return entry


def _rate_vs_measured(roof, peaks):
    if not peaks or roof is None:
        return
    if roof["bound"] == "hbm" and peaks.get("hbm_stream_read_1GiB_GBs"):
        roof["frac_of_measured_stream"] = round(roof["achieved"] / peaks["hbm_stream_read_1GiB_GBs"], 4)
        roof["frac_of_measured_stream_52MB"] = round(roof["achieved"] / peaks["hbm_stream_read_52MB_GBs"], 4)
        roof["frac_of_measured_stream_52MB_b2b"] = round(roof["achieved"] / peaks["hbm_stream_read_52MB_b2b_GBs"], 4)
    elif roof["bound"] == "mfma" and peaks.get("mfma_bf16_TFLOPs"):
        roof["frac_of_measured_mfma"] = round(roof["achieved"] / peaks["mfma_bf16_TFLOPs"], 4)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only: the layer runs on a single MI355X and "
                                   "has no multi-GPU path; run with --gpus 1"}))
        sys.exit(2)

    import workload

    head = args.workload or DEFAULT_WORKLOAD
    extra = [] if (args.workload or args.no_configs or args.peaks_only) else [n for n, _ in CONFIGS]
    sp = workload.spec(head)
    if args.experts != "arrays" and (sp.bits not in (2, 4) or sp.group != 128):
        print(json.dumps({"error": "the address-table entry points take INT4 and 2-bit with groups of 128"}))
        sys.exit(2)
    cpu = {} if args.peaks_only else {n: start_cpu_baseline(args, n, i) for i, n in enumerate([head] + extra)}

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    peaks = None if args.no_peaks else measure_peaks(dev)
    if args.peaks_only:
        print(json.dumps({"peaks": peaks}), flush=True)
        return
    line_head = run_workload(head, args, dev, args.steps, args.warmup)
    print(f"[bench] {head}: {line_head['value']} tokens/s", flush=True)
    configs = {}
    for n in extra:
        esp = workload.spec(n)
        k = max(args.steps, MIN_STEPS_DECODE if esp.T <= 512 else MIN_STEPS_PREFILL)
        configs[n] = run_workload(n, args, dev, k, max(args.warmup, 10))
        print(f"[bench] {n}: {configs[n]['value']} tokens/s", flush=True)
    line = {
        "metric": METRIC, "value": line_head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": line_head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": line_head["config"],
        "roofline": line_head["roofline"], "cpu_baseline": finish_cpu_baseline(cpu.get(head)),
        "step_ms": line_head["step_ms"],
    }
    if "ffn_stage" in line_head:
        line["ffn_stage"] = line_head["ffn_stage"]
    _rate_vs_measured(line["roofline"], peaks)
    _rate_vs_measured(line.get("ffn_stage"), peaks)
    for n, e in configs.items():
        e["cpu_baseline"] = finish_cpu_baseline(cpu.get(n))
        _rate_vs_measured(e["roofline"], peaks)
        _rate_vs_measured(e.get("ffn_stage"), peaks)
    if configs:
        line["configs"] = configs
    if peaks:
        line["peaks"] = peaks
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
