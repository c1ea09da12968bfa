"""moe_layer_w4a16_noalloc (the layer on the library's own device scratch) against
moe_layer_w4a16 with a caller workspace: y, ids and gates bit for bit, on two calls
in a row, the second with a smaller batch, and again after it."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import bit_quantized_moe_amd as bq
import workload
from gpu_util import to_dev, weights_to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(T, seed, H=4096, I=1024, E=256, k=8):
    sp = workload.spec("tiny_t4_h256_e8_k2_i128_int4", T=T, H=H, I=I, E=E, k=k, seed=seed)
    inp = workload.make_layer_inputs(sp)
    return sp, inp


def _noalloc(sp, x, wr, bias, wd):
    """Through the C ABI directly: outputs allocated here, no workspace anywhere."""
    T = x.shape[0]
    y = torch.empty((T, sp.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, sp.k), dtype=torch.int32, device="cuda")
    g = torch.empty((T, sp.k), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    s = bq.lib().moe_layer_w4a16_noalloc(x.data_ptr(), wr.data_ptr(), bias.data_ptr() if bias is not None else None,
                                         T, sp.H, sp.E, sp.k, sp.I, wd["w13_codes"].data_ptr(),
                                         wd["w13_scales"].data_ptr(), wd["w2_codes"].data_ptr(),
                                         wd["w2_scales"].data_ptr(), y.data_ptr(), ids.data_ptr(), g.data_ptr(), st)
    assert s == 0, bq.lib().moe_last_error()
    return y, ids, g


@pytest.mark.parametrize("shape", ["full", "small"])
def test_noalloc_layer_matches_workspace_layer(shape):
    dims = dict(full=dict(H=4096, I=1024, E=256, k=8), small=dict(H=512, I=256, E=16, k=4))[shape]
    ws = bq.Workspaces("cuda")
    for T, seed in ((16, 8100), (1, 8101), (5, 8102)):          # second call smaller than the first, then larger
        say(f"[gpu-test] noalloc layer {shape} T={T}")
        sp, inp = _inputs(T, seed, **dims)
        wd = weights_to_dev(inp.weights)
        x, wr = to_dev(inp.x), to_dev(inp.w_router)
        bias = torch.tensor(np.linspace(0.02, -0.02, sp.E, dtype=np.float32), device="cuda")
        y0, i0, g0 = bq.layer(x, wr, bias, wd, sp.k, 4, sp.I, ws=ws, want_routing=True)
        y1, i1, g1 = _noalloc(sp, x, wr, bias, wd)
        torch.cuda.synchronize()
        assert torch.equal(i0, i1), T
        assert torch.equal(g0.view(torch.int32), g1.view(torch.int32)), T
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), T
        say(f"    T={T}: bit-exact with the workspace entry point")
    ws.check()


def test_noalloc_rejects_oversized_shape():
    sp, inp = _inputs(1, 8103, H=512, I=256, E=16, k=4)
    # T*k = 256 rows at H = 4096, I = 4096: a workspace of about 16 MiB (rejected before any launch,
    # so the weight arrays are never read)
    x = torch.zeros((16, 4096), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((16, 4096), dtype=torch.bfloat16, device="cuda")
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    y = torch.empty((16, 4096), dtype=torch.bfloat16, device="cuda")
    s = bq.lib().moe_layer_w4a16_noalloc(x.data_ptr(), wr.data_ptr(), None, 16, 4096, 16, 16, 4096, dummy.data_ptr(),
                                         dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(), y.data_ptr(), None,
                                         None, torch.cuda.current_stream().cuda_stream)
    assert s == 2 and b"scratch" in bq.lib().moe_last_error()
