"""Times the CPU oracle on a bounded sample of a workload (TEST/BENCH INFRASTRUCTURE ONLY).

Run as a child process by bench.py's CPU-baseline leg:

    python -m oracle.cpu_baseline --workload NAME --seconds 12 [--core C]

It pins itself to one core (the last one it may run on, or --core), keeps
BLAS single-threaded, builds the same seeded inputs as the benchmark and
times the unmodified oracle.  Prints one JSON object.

Samples:
  * batches of up to 64 tokens (decode, verify): whole-layer oracle calls
    (O1..O8, including unpack and dequant of the touched experts) on the
    workload's tokens, repeated until the time budget is spent;
  * prefill chunks: routing, top-k and permutation of every token (O1..O4),
    then the expert FFN (O5..O7) of one expert in eight (ids = 3 mod 8, all of
    their rows), then their combine share.  tokens/s = (sampled rows / k) over
    the FFN time of the sample plus the routing time charged pro rata to the
    sampled rows (the FFN of one expert in eight is about a tenth of the
    oracle's whole-chunk time).
"""
from __future__ import annotations

import os

for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

import argparse  # noqa: E402
import json  # noqa: E402
import time  # noqa: E402


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--seconds", type=float, default=12.0)
    ap.add_argument("--core", type=int, default=-1, help="core to pin to (default: the last allowed one)")
    a = ap.parse_args()

    allowed = sorted(os.sched_getaffinity(0))
    cpu = allowed[a.core % len(allowed)] if a.core >= 0 else allowed[-1]
    os.sched_setaffinity(0, {cpu})

    import numpy as np

    import workload
    from oracle import moe_oracle as O

    sp = workload.spec(a.workload)
    w_r, bias = workload.make_router(sp)
    weights = workload.make_weight_set(sp, 0)
    if sp.T <= 64:
        xs = [workload.make_x(sp, s) for s in range(min(sp.n_sets, 4))]
        calls = tokens = 0
        t0 = time.perf_counter()
        while True:
            x = xs[calls % len(xs)]
            if sp.nvfp4:
                O.moe_layer_nvfp4(x, w_r, bias, weights, sp.k, sp.I, sp.nv_gx, sp.nv_gh)
            else:
                O.moe_layer(x, w_r, bias, weights, sp.k, sp.bits, sp.I, group=sp.group)
            calls += 1
            tokens += sp.T
            el = time.perf_counter() - t0
            if el >= a.seconds:
                break
        value = tokens / el
        sample = (f"{calls} whole-layer oracle calls of {sp.T} token(s) each (O1-O8, incl. unpack and dequant "
                  f"of the touched experts, one weight set), {el:.1f} s on 1 core")
    else:
        x = workload.make_x(sp, 0)
        t0 = time.perf_counter()
        logits = O.router_logits(x, w_r, bias)
        ids, gates = O.topk_softmax(logits, sp.k)
        off, srt, rp, act = O.permute(ids, sp.E)
        t_route = time.perf_counter() - t0
        experts = [e for e in range(3, sp.E, 8) if off[e + 1] > off[e]]
        t1 = time.perf_counter()
        y_perm = O.expert_ffn(x, off, srt, sp.k, weights, sp.bits, sp.I, experts=experts, group=sp.group)
        rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
        part = y_perm[rows] * gates.ravel()[srt[rows]][:, None]   # their share of the combine
        t_ffn = time.perf_counter() - t1
        n_rows = int(rows.size)
        el = t_ffn + t_route * n_rows / (sp.T * sp.k)
        value = (n_rows / sp.k) / el
        sample = (f"routing of all {sp.T} tokens ({t_route:.1f} s, charged pro rata) and the expert FFN + combine "
                  f"share of {len(experts)} of {int(act[0])} active experts (ids 3 mod 8, {n_rows} of "
                  f"{sp.T * sp.k} rows, {t_ffn:.1f} s) on 1 core")
        del part
    print(json.dumps({
        "value": value, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": sample, "host_cpus": os.cpu_count(),
    }))


if __name__ == "__main__":
    main()
