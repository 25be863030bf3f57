"""GPU parity: trellis_decode_tiles and had128_scale against the CPU oracle.

Decoded weights must be bit-exact (fp16 codebook values); exported states must equal the
oracle's and satisfy the trellis overlap invariant."""
import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import as_u16, log_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,n_in,n_out", [
    (2, 512, 256),    # the single-matrix workload shape
    (3, 48, 80),      # ragged: tile counts not multiples of 8
    (4, 160, 272),
    (2, 16, 16),      # one tile
    (3, 256, 384),
    (4, 128, 2048),
])
def test_decode_bit_exact_and_states(K, n_in, n_out):
    log_case(f"decode K={K} {n_in}x{n_out}")
    lin = synth.make_linear(np.random.SeedSequence([K, n_in, n_out]), K, n_in, n_out)
    w, st = tb.trellis_decode_tiles(to_dev(lin.code), K, want_states=True)
    torch.cuda.synchronize()
    ref = O.decode_tiles(lin.code, K)
    assert np.array_equal(as_u16(w), ref.view(np.uint16))
    ref_st = O.tile_states(lin.code, K)
    got_st = as_u16(st)
    assert np.array_equal(got_st, ref_st)
    lo = got_st.astype(np.int64) & ((1 << (16 - K)) - 1)
    assert np.array_equal(lo, np.roll(got_st.astype(np.int64), -1, axis=-1) >> K)


def test_decode_single_k2_workload():
    wl = synth.single_k2(0)
    lin = wl.layers["w"]
    w, _ = tb.trellis_decode_tiles(to_dev(lin.code), 2)
    assert np.array_equal(as_u16(w), O.decode_tiles(lin.code, 2).view(np.uint16))


def test_decode_deterministic():
    lin = synth.make_linear(np.random.SeedSequence(77), 3, 256, 256)
    c = to_dev(lin.code)
    a, _ = tb.trellis_decode_tiles(c, 3)
    b, _ = tb.trellis_decode_tiles(c, 3)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("post", [False, True])
@pytest.mark.parametrize("xdt,ydt", [(torch.float16, torch.float16), (torch.float32, torch.float32),
                                     (torch.float16, torch.float32), (torch.float32, torch.float16)])
def test_had128_scale(post, xdt, ydt):
    rng = np.random.default_rng(3)
    rows, n = 5, 384
    x = rng.standard_normal((rows, n)).astype(np.float16 if xdt == torch.float16 else np.float32)
    r = rng.uniform(0.5, 1.5, n).astype(np.float16)
    s = rng.normal(1, 0.02, n).astype(np.float32)
    y = tb.had128_scale(to_dev(x), to_dev(r), to_dev(s), post=post, out_dtype=ydt)
    sc = O.side_scale(r, s)
    ref = O.had_blocks(x.astype(np.float64)) * sc if post else O.had_blocks(x.astype(np.float64) * sc)
    got = y.cpu().numpy().astype(np.float64)
    tol = 1e-3 if ydt == torch.float16 else 1e-6
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < tol


def test_had128_in_place_and_no_scales():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    t = to_dev(x)
    tb.had128_scale(t, out=t)
    ref = O.had_blocks(x.astype(np.float64))
    assert np.abs(t.cpu().numpy() - ref).max() < 1e-5
    # applying twice is the identity (H is its own inverse)
    tb.had128_scale(t, out=t)
    assert np.abs(t.cpu().numpy() - x).max() < 1e-5


def test_workspace_too_small_launches_nothing():
    lin = synth.single_k2(0).layers["w"]
    L = tb.TrellisLinear.from_host(lin).c()
    import ctypes
    y = torch.full((1, 256), 7.0, dtype=torch.float16, device="cuda")
    x = torch.zeros((1, 512), dtype=torch.float16, device="cuda")
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    st = tb.lib().trellis_gemv(ctypes.byref(L), x.data_ptr(), 1, y.data_ptr(), ws.data_ptr(), 256,
                               torch.cuda.current_stream().cuda_stream)
    assert st == -3
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("post", [False, True])
def test_had128_scale_unaligned_operands(post):
    """Operands only 2-byte aligned take the per-element kernel; both kernels agree with the
    oracle (and 5 x 3 blocks leave a partial group of the vectorised kernel)."""
    rng = np.random.default_rng(7)
    rows, n = 5, 384
    x = rng.standard_normal((rows, n)).astype(np.float16)
    r = rng.uniform(0.5, 1.5, n).astype(np.float16)
    s = rng.normal(1, 0.02, n).astype(np.float32)
    sc = O.side_scale(r, s)
    ref = O.had_blocks(x.astype(np.float64)) * sc if post else O.had_blocks(x.astype(np.float64) * sc)
    buf = torch.empty(rows * n + 1, dtype=torch.float16, device="cuda")
    xu = buf[1:].view(rows, n)
    xu.copy_(to_dev(x))
    ybuf = torch.empty(rows * n + 1, dtype=torch.float16, device="cuda")
    yu = ybuf[1:].view(rows, n)
    tb.had128_scale(xu, to_dev(r), to_dev(s), post=post, out=yu)
    ya = tb.had128_scale(to_dev(x), to_dev(r), to_dev(s), post=post)
    torch.cuda.synchronize()
    for y in (yu, ya):
        got = y.cpu().numpy().astype(np.float64)
        assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-3
