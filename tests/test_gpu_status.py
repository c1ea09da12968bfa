"""Bounded waits that give up are reported to the caller (moe_workspace_status).

The timeout is forced from the host with a zero spin limit: every wait then
gives up at its first look, the kernel still runs to its end (each give-up
path keeps its reads and writes inside the call's buffers) and the sticky
flag must come back through the C ABI.  Then the default limit is restored,
the workspace zeroed, and the same call must be right again.
"""
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_amd as bq
import oracle
import workload
from gpu_util import bf16_np_to_f32, to_dev, to_np, weights_to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_preset_flag_is_reported_and_cleared():
    say("[gpu-test] preset flag")
    ws = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    assert bq.workspace_status(ws) == 0
    ws.view(torch.int32)[2] = bq.WS_WAIT_TIMEOUT
    assert bq.workspace_status(ws, clear=False) == bq.WS_WAIT_TIMEOUT
    assert bq.workspace_status(ws, clear=True) == bq.WS_WAIT_TIMEOUT
    assert bq.workspace_status(ws) == 0
    assert int(ws.view(torch.int32).abs().sum()) == 0
    w = bq.Workspaces("cuda")
    w.get("layer", 8192).view(torch.int32)[2] = 1
    with pytest.raises(bq.MoEError, match="timed out"):
        w.check()
    w.check()                                           # cleared and zeroed by the first check


def test_layer_wait_timeout_reported_then_recovers():
    sp = workload.spec("decode_t1_h4096_e256_k8_i1024_int4")
    w_r, bias = workload.make_router(sp)
    inp = workload.LayerInputs(sp, workload.make_x(sp, 0), w_r, bias, workload.make_weight_set(sp, 0))
    wd = weights_to_dev(inp.weights)
    x, wr = to_dev(inp.x), to_dev(w_r)
    ws = bq.Workspaces("cuda")
    say("[gpu-test] layer T=1 with a zero spin limit")
    prev = bq.set_wait_limit(0)
    try:
        bq.layer(x, wr, None, wd, sp.k, sp.bits, sp.I, ws=ws)
        torch.cuda.synchronize()
    finally:
        bq.set_wait_limit(-1)
    assert prev == 1 << 22
    flags = bq.workspace_status(ws._bufs["layer"], clear=False)
    say(f"    flags after the forced timeout: {flags}")
    assert flags & bq.WS_WAIT_TIMEOUT
    with pytest.raises(bq.MoEError, match="timed out"):
        ws.check()                                      # clears the flags and zeroes the workspace
    say("[gpu-test] layer T=1 with the default limit")
    y = bq.layer(x, wr, None, wd, sp.k, sp.bits, sp.I, ws=ws)
    ws.check()
    ref = oracle.moe_layer(inp.x, inp.w_router, None, inp.weights, sp.k, sp.bits, sp.I)
    err = oracle.rel_fro(bf16_np_to_f32(to_np(y)), ref["y"])
    say(f"    y rel-fro {err:.2e}")
    assert err <= 2e-2
    torch.cuda.synchronize()
    assert int(ws._bufs["layer"].view(torch.int32).abs().sum()) == 0
