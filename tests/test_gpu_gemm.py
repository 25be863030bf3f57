"""GPU parity: trellis_gemm (prefill) against the fp64 CPU oracle, within 2e-3 relative L2."""
import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, dev_linear, log_case, oracle_forward_full, rel_l2, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("M,n_in,n_out", [(300, 256, 384), (1, 128, 128), (256, 512, 256), (17, 384, 128)])
def test_gemm_small_shapes(K, M, n_in, n_out):
    log_case(f"gemm K={K} M={M} {n_in}x{n_out}")
    lin = synth.make_linear(np.random.SeedSequence([K, M, n_in, n_out]), K, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([M, 2]), M, n_in)
    y = tb.trellis_gemm(dev_linear(lin), to_dev(x))
    torch.cuda.synchronize()
    ref = O.forward_linear(lin, x)
    assert rel_l2(y.cpu().numpy(), ref) < REL_L2_TOL


@pytest.mark.parametrize("wgs", [1, 3, 7, 16, 61])
def test_gemm_stream_k_splits(wgs, monkeypatch):
    """Forced workgroup counts move the range boundaries: one range over every tile, ranges
    over several tiles, ranges inside one tile, one k-step pair per range.  Every split of
    the k-sum must still give the oracle's product (M = 300: a ragged second row band)."""
    monkeypatch.setenv("TRELLIS_GEMM_WGS", str(wgs))
    log_case(f"gemm stream-K wgs={wgs}")
    lin = synth.make_linear(np.random.SeedSequence([77, wgs]), 3, 384, 512)
    x = synth.make_x(np.random.SeedSequence(78), 300, 384)
    y = tb.trellis_gemm(dev_linear(lin), to_dev(x))
    torch.cuda.synchronize()
    ref = O.forward_linear(lin, x)
    assert rel_l2(y.cpu().numpy(), ref) < REL_L2_TOL


def _offset_copy(a: np.ndarray) -> torch.Tensor:
    """The same values one element past an allocation's start (2- or 4-byte aligned only)."""
    buf = torch.empty(a.size + 1, dtype=torch.from_numpy(a).dtype, device="cuda")
    buf[1:] = torch.from_numpy(a).cuda()
    return buf[1:]


def test_gemm_unaligned_side_vectors():
    """rin/s_in that are only naturally aligned take the element-load rotation."""
    lin = synth.make_linear(np.random.SeedSequence(41), 2, 256, 256)
    x = synth.make_x(np.random.SeedSequence(42), 40, 256)
    L = tb.TrellisLinear(torch.from_numpy(lin.code).cuda(), _offset_copy(lin.rin), _offset_copy(lin.rout),
                         _offset_copy(lin.s_in), _offset_copy(lin.s_out), lin.K)
    assert L.rin.data_ptr() % 16 != 0 and L.s_in.data_ptr() % 16 != 0
    y = tb.trellis_gemm(L, to_dev(x))
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), O.forward_linear(lin, x)) < REL_L2_TOL


def test_gemm_prefill_full_size_whole_output():
    """K3 5120 -> 17408 with M = 2048 (the prefill workload): every one of the 2048 x 17408
    outputs against the oracle (fp64 product of the decoded matrix)."""
    log_case("gemm prefill full size")
    wl = synth.prefill(0)
    lin, x = wl.layers["w"], wl.xs["w"]
    y = tb.trellis_gemm(dev_linear(lin), to_dev(x))
    torch.cuda.synchronize()
    ref = oracle_forward_full(("prefill", "w"), lin, x)
    yn = y.cpu().numpy()
    assert rel_l2(yn, ref) < REL_L2_TOL
    # and no row band or column block is off on its own
    for r0 in range(0, 2048, 512):
        assert rel_l2(yn[r0:r0 + 512], ref[r0:r0 + 512]) < REL_L2_TOL, r0


def test_gemm_matches_gemv_rows():
    """The prefill path and the small-batch path compute the same product."""
    lin = synth.make_linear(np.random.SeedSequence(31), 3, 512, 384)
    x = synth.make_x(np.random.SeedSequence(32), 8, 512)
    L = dev_linear(lin)
    yg = tb.trellis_gemm(L, to_dev(x)).cpu().numpy()
    yv = tb.trellis_gemv(L, to_dev(x)).cpu().numpy()
    assert rel_l2(yg, yv) < 1e-3


@pytest.mark.parametrize("M,n_in,n_out", [(17, 256, 384), (300, 128, 256), (513, 128, 128)])
def test_gemm_writes_only_m_rows(M, n_in, n_out):
    """The output rows past M (the tile's padding) are never written: y sits at the start of
    a larger buffer whose guard rows must keep their values."""
    log_case(f"gemm guard rows M={M} {n_in}x{n_out}")
    lin = synth.make_linear(np.random.SeedSequence([7, M, n_in, n_out]), 3, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([M, 9]), M, n_in)
    big = torch.full((M + 64, n_out), 12345.0, dtype=torch.float16, device="cuda")
    y = tb.trellis_gemm(dev_linear(lin), to_dev(x), out=big[:M])
    torch.cuda.synchronize()
    assert y.data_ptr() == big.data_ptr()
    assert bool((big[M:] == 12345.0).all())
    assert rel_l2(big[:M].cpu().numpy(), O.forward_linear(lin, x)) < REL_L2_TOL
