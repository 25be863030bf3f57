"""GPU parity of the FP8 variant (cb = 2, the E4M3 codebook) against the CPU oracle.

trellis_decode_tiles_e4m3 must be bit-exact over every one of the 65 536 states.
trellis_gemm_fp8 is compared with the oracle's FP8 prefill (the same per-row E4M3
quantisation of the rotated activations, then fp64 arithmetic) within 2e-3 relative L2:
E4M3 products are exact in the fp32 accumulator, so what remains is the accumulation order,
the fp16 output and the rare activation code that the fp32 rotation puts on the other side
of a rounding boundary than the fp64 one."""
import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, log_case, oracle_forward_full, rel_l2, to_dev, worst_block_rel_l2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [2, 3, 4])
def test_decode_e4m3_bit_exact_all_states(K):
    log_case(f"decode e4m3 K={K}")
    lin = synth.make_linear(np.random.SeedSequence([50, K]), K, 1024, 2048)
    st = O.tile_states(lin.code, K)
    assert np.unique(st).size == 1 << 16  # every state occurs
    w8 = tb.trellis_decode_tiles_e4m3(to_dev(lin.code), K)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(w8.cpu().numpy(), O.decode_tiles_e4m3(lin.code, K))


def _fp8_linear(seed, K, n_in, n_out):
    lin = synth.make_linear(np.random.SeedSequence(seed), K, n_in, n_out)
    lin.cb = 2
    return lin


def _gemm_fp8_np(lin, x):
    y = tb.trellis_gemm_fp8(tb.TrellisLinear.from_host(lin), to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("M,n_in,n_out", [(1, 128, 128), (37, 384, 256), (600, 1024, 384), (513, 640, 128)])
def test_gemm_fp8_small(K, M, n_in, n_out):
    log_case(f"gemm fp8 K={K} M={M} {n_in}x{n_out}")
    lin = _fp8_linear([51, K, M, n_in, n_out], K, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([52, M]), M, n_in)
    y = _gemm_fp8_np(lin, x)
    ref = O.forward_linear(lin, x, act_e4m3=True)
    assert rel_l2(y, ref) < REL_L2_TOL


@pytest.mark.parametrize("wgs", ["3", "7", "50"])
def test_gemm_fp8_split_tiles(monkeypatch, wgs):
    """Few workgroups: tiles split between two and among several ranges."""
    log_case(f"gemm fp8 wgs={wgs}")
    monkeypatch.setenv("TRELLIS_GEMM_WGS", wgs)
    lin = _fp8_linear([53, 3], 3, 1152, 384)
    x = synth.make_x(np.random.SeedSequence(54), 700, 1152)
    assert rel_l2(_gemm_fp8_np(lin, x), O.forward_linear(lin, x, act_e4m3=True)) < REL_L2_TOL


def test_gemm_fp8_zero_rows_and_determinism():
    lin = _fp8_linear([55, 2], 2, 256, 256)
    x = synth.make_x(np.random.SeedSequence(56), 40, 256)
    x[[0, 17, 39]] = 0
    L = tb.TrellisLinear.from_host(lin)
    xd = to_dev(x)
    y1 = tb.trellis_gemm_fp8(L, xd).clone()
    y2 = tb.trellis_gemm_fp8(L, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y = y1.cpu().numpy()
    assert np.all(y[[0, 17, 39]] == 0)
    assert rel_l2(y, O.forward_linear(lin, x, act_e4m3=True)) < REL_L2_TOL


def test_gemm_fp8_prefill_full_size():
    """K3 5120 -> 17408, M = 2048 (the prefill shape): every one of the 2048 x 17408 outputs
    against the oracle's FP8 prefill, and every 512-row band of every column block."""
    log_case("gemm fp8 prefill full size")
    lin = _fp8_linear([57], 3, 5120, 17408)
    x = synth.make_x(np.random.SeedSequence(58), 2048, 5120)
    y = _gemm_fp8_np(lin, x)
    ref = oracle_forward_full(("fp8 prefill", 57), lin, x, act_e4m3=True)
    assert rel_l2(y, ref) < REL_L2_TOL
    assert worst_block_rel_l2(y, ref) < REL_L2_TOL
    # the FP8 path against the unquantised activations: the E4M3 rounding of xh costs a
    # few percent, as the oracle's own band says
    exact = oracle_forward_full(("fp8 prefill", 57), lin, x[:64])
    assert 0.005 < rel_l2(y[:64], exact) < 0.05


# ------------------------------------------------------------------------------------------
# The E4M3 codebook in the fp16-activation products (GEMV, MoE, MLP, prefill)
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("n_in,n_out,B", [(384, 640, 1), (1152, 256, 3), (640, 384, 8)])
def test_gemv_e4m3_codebook(K, n_in, n_out, B):
    log_case(f"gemv e4m3 K={K} {n_in}x{n_out} B={B}")
    lin = _fp8_linear([60, K, n_in, n_out, B], K, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([61, B]), B, n_in)
    y = tb.trellis_gemv(tb.TrellisLinear.from_host(lin), to_dev(x))
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), O.forward_linear(lin, x)) < REL_L2_TOL


def test_gemv_e4m3_codebook_full_size():
    """up_proj shape K3 5120 -> 17408 with the E4M3 codebook, batch 1 and 8: the whole
    output and every column block."""
    log_case("gemv e4m3 full size")
    lin = _fp8_linear([62], 3, 5120, 17408)
    L = tb.TrellisLinear.from_host(lin)
    for B in (1, 8):
        x = synth.make_x(np.random.SeedSequence([63, B]), B, 5120)
        y = tb.trellis_gemv(L, to_dev(x))
        torch.cuda.synchronize()
        y = y.cpu().numpy()
        ref = oracle_forward_full(("e4m3 gemv", 62), lin, x)
        assert rel_l2(y, ref) < REL_L2_TOL, B
        assert worst_block_rel_l2(y, ref) < REL_L2_TOL, B


def test_moe_table_mixing_codebooks():
    lins = []
    for e, (K, cb) in enumerate([(2, 1), (3, 2), (4, 2), (2, 2), (3, 1), (4, 1)]):
        l = synth.make_linear(np.random.SeedSequence([64, e]), K, 256, 384)
        l.cb = cb
        lins.append(l)
    table = tb.ExpertTable([tb.TrellisLinear.from_host(l) for l in lins])
    routed = np.array([1, 0, 5, 2, 3, 2], np.int32)
    x = synth.make_x(np.random.SeedSequence(65), 1, 256)
    ws = torch.zeros(table.workspace_bytes(len(routed)), dtype=torch.uint8, device="cuda")  # own error word
    y = tb.trellis_moe_gemv(table, to_dev(routed), to_dev(x[0]), False, ws=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    for k, e in enumerate(routed):
        assert rel_l2(y[k], O.forward_linear(lins[e], x)[0]) < REL_L2_TOL, (k, e)
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_mlp_with_e4m3_slices():
    """A routed MLP whose gate/up slices and down matrices mix the two codebooks."""
    layer = synth.moe_mlp_layer(7, n_experts=4, hidden=256, inter=256, halves=2)
    for e in range(4):
        layer.gate[e][e % 2].cb = 2
        layer.up[e][1 - e % 2].cb = 2
        if e % 2:
            layer.down[e].cb = 2
    tables = tb.MoEMLPTables.from_host(layer)
    routed, w = [3, 0, 1], [0.5, 0.25, 0.25]
    x = synth.make_x(np.random.SeedSequence(66), 1, 256)
    y = tb.trellis_moe_mlp(tables, to_dev(np.array(routed, np.int32)), to_dev(np.array(w, np.float32)),
                           to_dev(x[0]), tables.r_hidden_in, tables.s_hidden_in, tables.r_hidden_out,
                           tables.s_hidden_out)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), O.moe_mlp_forward(layer, routed, w, x)) < REL_L2_TOL


@pytest.mark.parametrize("K", [2, 3, 4])
def test_gemm_fp16_e4m3_codebook(K):
    """trellis_gemm (fp16 activations) on E4M3 weights: the cb = 2 forward, no activation
    quantisation."""
    lin = _fp8_linear([67, K], K, 640, 384)
    x = synth.make_x(np.random.SeedSequence(68), 300, 640)
    y = tb.trellis_gemm(tb.TrellisLinear.from_host(lin), to_dev(x))
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), O.forward_linear(lin, x)) < REL_L2_TOL
