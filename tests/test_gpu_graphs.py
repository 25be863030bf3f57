"""Entry points captured in HIP graphs: every replay, with other eager work on the same
workspace and synchronisations in between, must reproduce the eager result bitwise.
(The benchmark times the products inside graphs; nothing in them records a memset.)"""
import numpy as np
import pytest
import torch

from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import log_case, to_dev

pytestmark = pytest.mark.gpu


def _check_replays(fn, disturb, outs):
    fn()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(7.0)
        disturb()  # eager work on the same workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), f"replay {rep} differs from the eager result"


def test_graph_gemv_and_moe():
    log_case("graph gemv/moe")
    wl = synth.dense_mlp(0)
    gate, up, down = (tb.TrellisLinear.from_host(wl.layers[n]) for n in ("gate", "up", "down"))
    table = tb.ExpertTable([gate, up])
    routed = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    x = to_dev(wl.xs["gate"][0])
    xd = to_dev(wl.xs["down"])
    ws = torch.zeros(max(table.workspace_bytes(2), down.workspace_bytes(tb.TRELLIS_OP_GEMV, 1)),
                     dtype=torch.uint8, device="cuda")
    y_gu = torch.empty((2, 17408), dtype=torch.float16, device="cuda")
    y_d = torch.empty((1, 5120), dtype=torch.float16, device="cuda")
    y_x = torch.empty((1, 5120), dtype=torch.float16, device="cuda")

    def fn():
        tb.trellis_moe_gemv(table, routed, x, False, out=y_gu, ws=ws)
        tb.trellis_gemv(down, xd, out=y_d, ws=ws)

    xd2 = to_dev(synth.make_x(np.random.SeedSequence(5), 1, 17408))
    _check_replays(fn, lambda: tb.trellis_gemv(down, xd2, out=y_x, ws=ws), [y_gu, y_d])


def test_graph_moe_mlp():
    log_case("graph moe mlp")
    layer = synth.moe_mlp_layer(1, n_experts=16, hidden=768, inter=512, halves=4)
    tables = tb.MoEMLPTables.from_host(layer)
    routed = to_dev(np.array([3, 9, 0, 15, 7, 2, 11, 5], np.int32))
    w = to_dev(synth.moe_router_weights(1, 1)[0])
    x = to_dev(synth.make_x(np.random.SeedSequence(6), 1, 768)[0])
    ws = torch.zeros(tables.workspace_bytes(8), dtype=torch.uint8, device="cuda")
    y = torch.empty(768, dtype=torch.float16, device="cuda")
    act = torch.empty((8, 512), dtype=torch.float16, device="cuda")
    y2 = torch.empty(768, dtype=torch.float16, device="cuda")
    args = (tables.r_hidden_in, tables.s_hidden_in, tables.r_hidden_out, tables.s_hidden_out)

    def fn():
        tb.trellis_moe_mlp(tables, routed, w, x, *args, out=y, act=act, ws=ws)

    routed2 = to_dev(np.array([1, 4], np.int32))
    w2 = to_dev(np.array([0.3, 0.7], np.float32))
    _check_replays(fn, lambda: tb.trellis_moe_mlp(tables, routed2, w2, x, *args, out=y2, ws=ws), [y, act])


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_prefill(fp8):
    log_case(f"graph prefill fp8={fp8}")
    lin = synth.make_linear(np.random.SeedSequence(8), 3, 1024, 768)
    lin.cb = 2 if fp8 else 1
    L = tb.TrellisLinear.from_host(lin)
    x = to_dev(synth.make_x(np.random.SeedSequence(9), 700, 1024))
    x2 = to_dev(synth.make_x(np.random.SeedSequence(10), 300, 1024))
    f = tb.trellis_gemm_fp8 if fp8 else tb.trellis_gemm
    op = tb.TRELLIS_OP_GEMM_FP8 if fp8 else tb.TRELLIS_OP_GEMM
    ws = torch.zeros(L.workspace_bytes(op, 700), dtype=torch.uint8, device="cuda")
    y = torch.empty((700, 768), dtype=torch.float16, device="cuda")
    y2 = torch.empty((300, 768), dtype=torch.float16, device="cuda")
    _check_replays(lambda: f(L, x, out=y, ws=ws), lambda: f(L, x2, out=y2, ws=ws), [y])
