"""The allocation-free entry point (trellis_gemv_list_noalloc) against trellis_gemv_list:
called through the C ABI, two calls in a row (the second with a smaller input), each equal
to the workspace entry point's result."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, dev_linear, log_case, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _noalloc(layers, xs, B):
    ys = [torch.empty((B, l.out_features), dtype=torch.float16, device="cuda") for l in layers]
    items = tb._gemv_items(layers, [x.reshape(B, -1) for x in xs], ys)
    st = tb.lib().trellis_gemv_list_noalloc(items, len(layers), B, tb._stream())
    assert st == 0, tb.lib().trellis_last_error()
    return ys


def test_noalloc_matches_workspace_entry_point_twice():
    log_case("noalloc: large call then small call")
    # first call: the dense MLP step's three matrices at batch 2
    wl = synth.dense_mlp(0, batch=2)
    names = ["gate", "up", "down"]
    L1 = [dev_linear(wl.layers[n]) for n in names]
    x1 = [to_dev(wl.xs[n]) for n in names]
    a1 = _noalloc(L1, x1, 2)
    r1 = tb.trellis_gemv_list(L1, x1)
    # second call, smaller: two small layers at batch 1
    lins = [synth.make_linear(np.random.SeedSequence([80, i]), K, n_in, n_out)
            for i, (K, n_in, n_out) in enumerate([(2, 256, 384), (4, 640, 128)])]
    L2 = [dev_linear(l) for l in lins]
    xs2 = [synth.make_x(np.random.SeedSequence([81, i]), 1, l.in_features) for i, l in enumerate(lins)]
    x2 = [to_dev(x) for x in xs2]
    a2 = _noalloc(L2, x2, 1)
    r2 = tb.trellis_gemv_list(L2, x2)
    torch.cuda.synchronize()
    for a, r in zip(a1 + a2, r1 + r2):
        # the same kernels on the same geometry: the same bits
        assert torch.equal(a.view(torch.int16), r.view(torch.int16))
    for a, l, x in zip(a2, lins, xs2):
        assert rel_l2(a.cpu().numpy(), O.forward_linear(l, x)) < REL_L2_TOL


def test_noalloc_rejects_oversized_requests():
    """A request needing more scratch than the library holds fails before launching: one
    128-row layer with 8192 column blocks at batch 8 (every workgroup's share meets several
    column blocks, each with an 8-row partial)."""
    n_out = 128 * 8192
    big = [tb.TrellisLinear(torch.zeros((8, n_out // 16, 64), dtype=torch.int16, device="cuda"),
                            torch.ones(128, dtype=torch.float16, device="cuda"),
                            torch.ones(n_out, dtype=torch.float16, device="cuda"), None, None, 4)]
    x = [torch.zeros((8, 128), dtype=torch.float16, device="cuda")]
    y = [torch.empty((8, n_out), dtype=torch.float16, device="cuda")]
    need = tb.trellis_gemv_list_workspace_bytes(big, 8)
    assert need > 32 << 20, need
    items = tb._gemv_items(big, x, y)
    st = tb.lib().trellis_gemv_list_noalloc(items, 1, 8, tb._stream())
    assert st == -4 and b"scratch" in tb.lib().trellis_last_error()
