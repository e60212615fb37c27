"""qmoe_forward_noalloc, called through the C ABI, against qmoe_forward.

The no-allocation entry point runs the same dispatch and kernels as
qmoe_forward with the library's own device array as the workspace, so its
output must equal qmoe_forward's bit for bit. Two calls in a row on one
handle, the second with fewer tokens, check that what the first call left in
the shared array does not leak into the second; a size whose workspace would
exceed the array is refused before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import qmoe_inputs as qi
import quantized_mixture_experts_qmoe_amd as q
from tests.gpu_util import DEV, layer_for, say

pytestmark = pytest.mark.gpu


def _noalloc(layer, x, logits):
    out = torch.full_like(x, float("nan"))
    st = q.lib().qmoe_forward_noalloc(layer._h, ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(logits.data_ptr()),
                                      ctypes.c_void_p(out.data_ptr()), x.shape[0], q._stream())
    return st, out


def _tokens(spec, T, seed):
    t = qi.draw_tokens(spec, T, np.random.default_rng(seed), nseq=max(1, T // 50))
    return t.x.to(DEV), t.logits.to(DEV)


@pytest.mark.parametrize("sizes", [(300, 4), (256, 100), (4, 1), (24, 9)])
def test_noalloc_matches_forward(sizes):
    wl = qi.make_workload("decode", T=1)
    layer = layer_for(wl, 512)
    for i, T in enumerate(sizes):
        x, g = _tokens(wl.spec, T, 1000 + 17 * i + T)
        say(f"noalloc T={T} (call {i + 1} of {len(sizes)})")
        ref = layer(x, g, workspace=torch.empty(layer.workspace_size(T), dtype=torch.uint8,
                                                device=DEV))
        st, out = _noalloc(layer, x, g)
        torch.cuda.synchronize()
        assert st == 0, st
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), T
    assert layer.decode_errors() == 0


def test_noalloc_refuses_sizes_beyond_its_array():
    wl = qi.make_workload("decode", T=1)
    layer = layer_for(wl, 2048)
    T = 2048
    assert layer.workspace_size(T) > q.NOALLOC_WORKSPACE_BYTES
    x, g = _tokens(wl.spec, T, 5)
    st, out = _noalloc(layer, x, g)
    torch.cuda.synchronize()
    assert st == 3, st                                   # QMOE_ERR_WORKSPACE
    assert torch.isnan(out.float()).all()                # nothing was enqueued
    # the largest size that fits still runs and matches qmoe_forward
    n = max(t for t in range(1, T) if layer.workspace_size(t) <= q.NOALLOC_WORKSPACE_BYTES)
    say(f"noalloc largest size {n}")
    x, g = x[:n].contiguous(), g[:n].contiguous()
    ref = layer(x, g)
    st, out = _noalloc(layer, x, g)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(out.view(torch.int16), ref.view(torch.int16))
