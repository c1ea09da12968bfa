"""Times the CPU oracle on a bounded sample of a workload (TEST/BENCH INFRASTRUCTURE ONLY).

Run as a child process by bench.py's CPU-baseline leg:

    python -m oracle.cpu_baseline --workload NAME --seconds 12

It pins itself to one core, keeps BLAS single-threaded, builds the same seeded
inputs as the benchmark, and repeats whole-layer oracle calls (O1..O8) on
sampled tokens until the time budget is spent.  Prints one JSON object.
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
    ap.add_argument("--tokens-per-call", type=int, default=0, help="0: the workload's T, capped at 32")
    a = ap.parse_args()

    cpu = sorted(os.sched_getaffinity(0))[-1]
    os.sched_setaffinity(0, {cpu})

    import numpy as np

    import workload
    from oracle import moe_oracle as O

    sp = workload.spec(a.workload)
    w_r, bias = workload.make_router(sp)
    weights = workload.make_weight_set(sp, 0)
    n_tok = a.tokens_per_call or min(sp.T, 32)
    xs = [workload.make_x(sp, s) for s in range(min(sp.n_sets, 4))]

    calls = tokens = 0
    t0 = time.perf_counter()
    rng = np.random.default_rng(0)
    while True:
        x = xs[calls % len(xs)]
        tok = np.sort(rng.choice(sp.T, n_tok, replace=False)) if n_tok < sp.T else np.arange(sp.T)
        O.moe_layer_tokens(x, w_r, bias, weights, sp.k, sp.bits, sp.I, tok, group=sp.group)
        calls += 1
        tokens += len(tok)
        el = time.perf_counter() - t0
        if el >= a.seconds:
            break
    print(json.dumps({
        "value": tokens / el, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
        "sample": f"{calls} oracle layer calls of {n_tok} token(s) each (whole layer O1-O8, incl. unpack and "
                  f"dequant of the touched experts, one weight set), {el:.1f} s on 1 core",
        "seconds": el, "calls": calls, "host_cpus": os.cpu_count(),
    }))


if __name__ == "__main__":
    main()
