"""GPU parity: trellis_gemv, trellis_gemv_list and trellis_moe_gemv against the fp64 CPU
oracle.

Outputs must be within 2e-3 relative L2 of the oracle over each WHOLE output tensor,
including at the full sizes of the dense-MLP, small-batch and MoE workloads (the oracle
decodes each full-size matrix once per session, gpu_util.oracle_w_hat)."""
import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, dev_linear, log_case, oracle_forward_full, oracle_w_hat, rel_l2, to_dev

pytestmark = pytest.mark.gpu

RESERVED = 256 + 65536  # error word header + the small-batch counters at the start of a workspace


def _gemv_np(L, x):
    y = tb.trellis_gemv(L, to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _counters_zero(ws: torch.Tensor) -> bool:
    return bool((ws[256:RESERVED] == 0).all())


# ------------------------------------------------------------------------------------------
# Single layer
# ------------------------------------------------------------------------------------------

def test_gemv_single_k2_workload():
    wl = synth.single_k2(0)
    lin, x = wl.layers["w"], wl.xs["w"]
    y = _gemv_np(dev_linear(lin), x)
    assert rel_l2(y, O.forward_linear(lin, x)) < REL_L2_TOL


def test_single_k2_null_scales_every_product():
    """The single-matrix workload has s_in = s_out = 1 exactly, so passing NULL scales (the
    "all ones" branches of every kernel) must give the oracle's result -- and bitwise the
    result of passing the all-ones vectors -- through trellis_gemv, trellis_gemv_list,
    trellis_gemm and trellis_moe_gemv."""
    wl = synth.single_k2(0)
    lin, x = wl.layers["w"], wl.xs["w"]
    assert np.all(lin.s_in == 1.0) and np.all(lin.s_out == 1.0)
    ref = O.forward(lin.code, lin.K, lin.rin, lin.rout, None, None, x)
    Ln, L1 = dev_linear(lin, null_scales=True), dev_linear(lin)
    xd = to_dev(x)
    y_null = tb.trellis_gemv(Ln, xd).clone()
    y_ones = tb.trellis_gemv(L1, xd).clone()
    y_list = tb.trellis_gemv_list([Ln], [xd])[0]
    y_gemm = tb.trellis_gemm(Ln, xd)
    y_gemm1 = tb.trellis_gemm(L1, xd)
    table = tb.ExpertTable([Ln, Ln])
    y_moe = tb.trellis_moe_gemv(table, to_dev(np.array([1], np.int32)), xd[0], False)
    torch.cuda.synchronize()
    for name, y in (("gemv", y_null), ("list", y_list), ("gemm", y_gemm), ("moe", y_moe)):
        assert rel_l2(y.cpu().numpy(), ref) < REL_L2_TOL, name
    assert torch.equal(y_null.view(torch.int16), y_ones.view(torch.int16))
    assert torch.equal(y_gemm.view(torch.int16), y_gemm1.view(torch.int16))


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("n_in,n_out,B", [(384, 640, 1), (1152, 256, 3), (128, 128, 8), (640, 384, 5)])
def test_gemv_small_shapes(K, n_in, n_out, B):
    log_case(f"gemv K={K} {n_in}x{n_out} B={B}")
    lin = synth.make_linear(np.random.SeedSequence([K, n_in, n_out, B]), K, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([B, 1]), B, n_in)
    y = _gemv_np(dev_linear(lin), x)
    ref = O.forward_linear(lin, x)
    assert y.shape == ref.shape
    assert rel_l2(y, ref) < REL_L2_TOL
    for b in range(B):  # every batch row separately too
        assert rel_l2(y[b], ref[b]) < REL_L2_TOL


@pytest.mark.parametrize("wgs", ["3", "7", "1"])
def test_gemv_ranges_spanning_column_blocks(monkeypatch, wgs):
    """Few workgroups: each range covers several column blocks and cuts them mid-way, so the
    partials, the arrival counters and the last-arriver finish are exercised."""
    monkeypatch.setenv("TRELLIS_GEMV_WGS", wgs)
    log_case(f"gemv spanning wgs={wgs}")
    lin = synth.make_linear(np.random.SeedSequence(5), 3, 640, 896)
    x = synth.make_x(np.random.SeedSequence(6), 2, 640)
    y = _gemv_np(dev_linear(lin), x)
    assert rel_l2(y, O.forward_linear(lin, x)) < REL_L2_TOL


def test_gemv_back_to_back_deterministic():
    """Repeated calls reuse the workspace (counters reset by the finishing workgroups) and
    give identical bits (partials are added in workgroup order, whoever finishes)."""
    lin = synth.make_linear(np.random.SeedSequence(8), 2, 1024, 768)
    x = to_dev(synth.make_x(np.random.SeedSequence(9), 4, 1024))
    L = dev_linear(lin)
    ws = torch.zeros(L.workspace_bytes(tb.TRELLIS_OP_GEMV, 4), dtype=torch.uint8, device="cuda")
    ys = [tb.trellis_gemv(L, x, ws=ws).clone() for _ in range(4)]
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    assert _counters_zero(ws)
    ref = O.forward_linear(lin, x.cpu().numpy())
    assert rel_l2(ys[-1].cpu().numpy(), ref) < REL_L2_TOL


def _offset_copy(a: np.ndarray) -> torch.Tensor:
    """The same values one element past an allocation's start (2- or 4-byte aligned only)."""
    buf = torch.empty(a.size + 1, dtype=torch.from_numpy(a).dtype, device="cuda")
    buf[1:] = torch.from_numpy(a.reshape(-1)).cuda()
    return buf[1:].view(a.shape)


def test_gemv_unaligned_operands_take_the_element_path():
    """x, rin and s_in that are only naturally aligned take the element-load rotation; the
    16-byte path and it give the oracle's result."""
    lin = synth.make_linear(np.random.SeedSequence(18), 3, 640, 256)
    x = synth.make_x(np.random.SeedSequence(19), 3, 640)
    L = tb.TrellisLinear(to_dev(lin.code), _offset_copy(lin.rin), to_dev(lin.rout), _offset_copy(lin.s_in),
                         to_dev(lin.s_out), lin.K)
    xu = _offset_copy(x)
    assert xu.data_ptr() % 16 and L.rin.data_ptr() % 16 and L.s_in.data_ptr() % 16
    y = tb.trellis_gemv(L, xu).cpu().numpy()
    ya = _gemv_np(dev_linear(lin), x)
    ref = O.forward_linear(lin, x)
    assert rel_l2(y, ref) < REL_L2_TOL and rel_l2(ya, ref) < REL_L2_TOL


def test_gemv_zero_rows():
    """All-zero activation rows give exactly zero output rows; the other rows match."""
    lin = synth.make_linear(np.random.SeedSequence(14), 3, 768, 384)
    x = synth.make_x(np.random.SeedSequence(15), 4, 768)
    x[0] = 0
    x[2] = 0
    y = _gemv_np(dev_linear(lin), x)
    assert np.all(y[0] == 0) and np.all(y[2] == 0)
    ref = O.forward_linear(lin, x)
    assert rel_l2(y[[1, 3]], ref[[1, 3]]) < REL_L2_TOL


def test_gemv_large_dynamic_range():
    """Activations far from N(0, 1): a 128-block of constant 600 and a block with four
    +-3e4 outliers.  Their normalised rotations (and the product, here with small s_out)
    are finite in fp16, so the library must be too: it stores the rotated activations at
    2^-4 of the butterfly's sum, within a factor 2^-0.5 of the normalised value."""
    lin = synth.make_linear(np.random.SeedSequence(16), 2, 512, 256)
    lin.s_out = np.full(256, 1e-3, np.float32)
    x = synth.make_x(np.random.SeedSequence(17), 2, 512)
    x[0, 0:128] = 600.0
    x[1, 128 + np.array([3, 40, 77, 100])] = np.array([3e4, -3e4, 3e4, 3e4], np.float16)
    ref = O.forward_linear(lin, x)
    assert np.all(np.abs(ref) < 6e4)
    L = dev_linear(lin)
    for name, y in (("gemv", _gemv_np(L, x)), ("gemm", tb.trellis_gemm(L, to_dev(x)).cpu().numpy())):
        assert np.all(np.isfinite(y)), name
        assert rel_l2(y, ref) < REL_L2_TOL, name


# ------------------------------------------------------------------------------------------
# Lists of layers in one launch
# ------------------------------------------------------------------------------------------

def _mixed_layers(seed):
    specs = [(2, 1, 256, 384), (3, 1, 640, 128), (4, 2, 384, 512), (3, 2, 128, 256), (2, 1, 1024, 640)]
    return [synth.make_linear(np.random.SeedSequence([seed, i]), K, n_in, n_out)
            for i, (K, cb, n_in, n_out) in enumerate(specs)], [s[1] for s in specs]


@pytest.mark.parametrize("B", [1, 3, 8])
def test_gemv_list_mixed_shapes_widths_codebooks(B):
    """Five layers of different shapes, widths and codebooks in one launch: every output
    matches its own layer's oracle."""
    lins, cbs = _mixed_layers(B)
    for l, cb in zip(lins, cbs):
        l.cb = cb
    xs = [synth.make_x(np.random.SeedSequence([B, i, 3]), B, l.in_features) for i, l in enumerate(lins)]
    ys = tb.trellis_gemv_list([dev_linear(l) for l in lins], [to_dev(x) for x in xs])
    torch.cuda.synchronize()
    for i, (l, x, y) in enumerate(zip(lins, xs, ys)):
        assert rel_l2(y.cpu().numpy(), O.forward_linear(l, x)) < REL_L2_TOL, i


@pytest.mark.parametrize("wgs", [1, 2, 5, 13])
def test_gemv_list_few_workgroups(monkeypatch, wgs):
    """Forced workgroup counts: ranges cross problems and column blocks of different heights
    (each problem's blocks have its own number of input blocks)."""
    monkeypatch.setenv("TRELLIS_GEMV_WGS", str(wgs))
    lins, _ = _mixed_layers(40 + wgs)
    xs = [synth.make_x(np.random.SeedSequence([wgs, i]), 2, l.in_features) for i, l in enumerate(lins)]
    ws = torch.zeros(tb.trellis_gemv_list_workspace_bytes([dev_linear(l) for l in lins], 2), dtype=torch.uint8,
                     device="cuda")
    ys = tb.trellis_gemv_list([dev_linear(l) for l in lins], [to_dev(x) for x in xs], ws=ws)
    torch.cuda.synchronize()
    for i, (l, x, y) in enumerate(zip(lins, xs, ys)):
        assert rel_l2(y.cpu().numpy(), O.forward_linear(l, x)) < REL_L2_TOL, (wgs, i)
    assert _counters_zero(ws)


def test_gemv_list_uniform_width_kernel():
    """Layers sharing one width and codebook take the specialised kernel; a repeated call
    gives the same bits."""
    lins = [synth.make_linear(np.random.SeedSequence([70, i]), 3, n_in, n_out)
            for i, (n_in, n_out) in enumerate([(512, 256), (256, 1024), (1536, 128)])]
    xs = [to_dev(synth.make_x(np.random.SeedSequence([71, i]), 1, l.in_features)) for i, l in enumerate(lins)]
    Ls = [dev_linear(l) for l in lins]
    a = [y.clone() for y in tb.trellis_gemv_list(Ls, xs)]
    b = tb.trellis_gemv_list(Ls, xs)
    torch.cuda.synchronize()
    for i, l in enumerate(lins):
        assert torch.equal(a[i].view(torch.int16), b[i].view(torch.int16))
        assert rel_l2(a[i].cpu().numpy(), O.forward_linear(l, xs[i].cpu().numpy())) < REL_L2_TOL


# ------------------------------------------------------------------------------------------
# Full size: whole outputs
# ------------------------------------------------------------------------------------------

@pytest.fixture(scope="module")
def dense_wl():
    return synth.dense_mlp(0)


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_dense_mlp_decode_bit_exact_every_tile(dense_wl, which):
    """trellis_decode_tiles on the whole matrix equals the oracle's decode bit for bit."""
    log_case(f"decode dense MLP {which} full")
    lin = dense_wl.layers[which]
    w, _ = tb.trellis_decode_tiles(to_dev(lin.code), lin.K)
    got = w.cpu().numpy().view(np.uint16)
    ref = oracle_w_hat(("dense", which), lin).view(np.uint16)
    assert got.shape == ref.shape
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_dense_mlp_full_size_whole_output(dense_wl, which):
    log_case(f"gemv dense MLP {which} full")
    lin, x = dense_wl.layers[which], dense_wl.xs[which]
    y = _gemv_np(dev_linear(lin), x)
    assert rel_l2(y, oracle_forward_full(("dense", which), lin, x)) < REL_L2_TOL


def test_dense_step_one_list_launch_whole_outputs(dense_wl):
    """The benchmarked step: gate, up and down (each on its own input) as one launch."""
    log_case("dense step as one list launch")
    names = ["gate", "up", "down"]
    ys = tb.trellis_gemv_list([dev_linear(dense_wl.layers[n]) for n in names],
                              [to_dev(dense_wl.xs[n]) for n in names])
    torch.cuda.synchronize()
    for n, y in zip(names, ys):
        ref = oracle_forward_full(("dense", n), dense_wl.layers[n], dense_wl.xs[n])
        assert rel_l2(y.cpu().numpy(), ref) < REL_L2_TOL, n


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_small_batch_full_size_whole_output(B):
    """The small-batch workload at batch B: its three matrices as one list launch (and each
    alone), every output complete against the oracle."""
    log_case(f"small-batch full B={B}")
    wl = synth.small_batch(0, batch=B)
    names = ["qkv", "z", "out"]
    Ls = [dev_linear(wl.layers[n]) for n in names]
    ys = tb.trellis_gemv_list(Ls, [to_dev(wl.xs[n]) for n in names])
    torch.cuda.synchronize()
    for n, y, L in zip(names, ys, Ls):
        ref = oracle_forward_full(("small", n), wl.layers[n], wl.xs[n])
        assert rel_l2(y.cpu().numpy(), ref) < REL_L2_TOL, n
        if B in (1, 8):
            assert rel_l2(_gemv_np(L, wl.xs[n]), ref) < REL_L2_TOL, n


# ------------------------------------------------------------------------------------------
# MoE
# ------------------------------------------------------------------------------------------

def _moe_small(shared_side):
    rng = np.random.default_rng(12)
    Ks = [2, 3, 4, 2, 3, 4]
    n_in, n_out = 256, 384
    lins = [synth.make_linear(np.random.SeedSequence([40, e]), K, n_in, n_out) for e, K in enumerate(Ks)]
    shared_r = rng.uniform(0.5, 1.5, n_in if shared_side == 0 else n_out).astype(np.float16)
    shared_s = rng.normal(1, 0.02, shared_r.shape[0]).astype(np.float32)
    return lins, shared_r, shared_s


@pytest.mark.parametrize("shared_side,x_per_expert", [(0, False), (1, True), (-1, True), (-1, False)])
def test_moe_small(shared_side, x_per_expert):
    log_case(f"moe small side={shared_side} xpe={x_per_expert}")
    lins, sr, ss = _moe_small(shared_side)
    table = tb.ExpertTable([dev_linear(l) for l in lins], shared_side=shared_side)
    routed = np.array([5, 0, 3, 3, 1, 4, 2], np.int32)
    n = len(routed)
    x = synth.make_x(np.random.SeedSequence(13), n if x_per_expert else 1, 256)
    ws = torch.zeros(table.workspace_bytes(len(routed)), dtype=torch.uint8, device="cuda")  # own error word
    y = tb.trellis_moe_gemv(table, to_dev(routed), to_dev(x if x_per_expert else x[0]), x_per_expert,
                            to_dev(sr) if shared_side >= 0 else None, to_dev(ss) if shared_side >= 0 else None,
                            shared_side, ws=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    for k, e in enumerate(routed):
        l = lins[e]
        rin, s_in, rout, s_out = l.rin, l.s_in, l.rout, l.s_out
        if shared_side == 0:
            rin, s_in = sr, ss
        if shared_side == 1:
            rout, s_out = sr, ss
        xe = x[k:k + 1] if x_per_expert else x[0:1]
        ref = O.forward(l.code, l.K, rin, rout, s_in, s_out, xe)[0]
        assert rel_l2(y[k], ref) < REL_L2_TOL, (k, e)
    assert tb.error_word(ws) == 0
    assert _counters_zero(ws)


def _bad_table():
    lins, sr, ss = _moe_small(-1)
    devl = [dev_linear(l) for l in lins[:3]]
    table = tb.ExpertTable(devl)
    # corrupt entry 1's K on the device copy (the kernel must reject it, not decode it)
    raw = bytearray(table.table.cpu().numpy().tobytes())
    sz = len(raw) // 3
    raw[sz + 40:sz + 44] = (9).to_bytes(4, "little")  # K field of entry 1
    table.table = torch.frombuffer(raw, dtype=torch.uint8).cuda()
    return table


def test_moe_bad_entries_give_zero_rows_and_error_word():
    table = _bad_table()
    routed = to_dev(np.array([0, 1, 7, 2], np.int32))  # entry 1 bad K, id 7 out of range
    x = to_dev(synth.make_x(np.random.SeedSequence(3), 1, 256)[0])
    ws = torch.zeros(table.workspace_bytes(4), dtype=torch.uint8, device="cuda")
    y = tb.trellis_moe_gemv(table, routed, x, False, ws=ws)
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert np.all(yn[1] == 0) and np.all(yn[2] == 0)
    assert np.any(yn[0] != 0) and np.any(yn[3] != 0)
    assert tb.error_word(ws) == 1
    assert _counters_zero(ws)


def test_error_word_is_sticky_until_cleared():
    """The error word keeps a bad call's bit through later clean calls; after the caller
    clears it (a fill on the stream), a clean call leaves it zero."""
    table = _bad_table()
    x = to_dev(synth.make_x(np.random.SeedSequence(4), 1, 256)[0])
    ws = torch.zeros(table.workspace_bytes(2), dtype=torch.uint8, device="cuda")
    tb.trellis_moe_gemv(table, to_dev(np.array([1, 0], np.int32)), x, False, ws=ws)
    clean = to_dev(np.array([0, 2], np.int32))
    tb.trellis_moe_gemv(table, clean, x, False, ws=ws)
    assert tb.error_word(ws) == 1
    tb.clear_error_word(ws)
    y = tb.trellis_moe_gemv(table, clean, x, False, ws=ws)
    torch.cuda.synchronize()
    assert tb.error_word(ws) == 0
    assert np.all(np.any(y.cpu().numpy() != 0, axis=1))


def _moe_full(routing_seed):
    routed = synth.moe_routes(routing_seed, 1)[0]
    layer = synth.moe_layer(0, experts=routed.tolist())
    return routed, layer


@pytest.mark.parametrize("routing_seed", [0, 1])
def test_moe_glm_like_full_size_whole_outputs(routing_seed):
    """8 routed experts of the GLM-like layer (6144 <-> 2048, K per expert from 2/3/4): gate
    and up (16 products, one launch, shared hidden-side input vectors) and down (8 products
    on per-expert inputs, shared hidden-side output vectors).  Every output row complete
    against the oracle, for two routings."""
    routed, layer = _moe_full(routing_seed)
    log_case(f"moe full routed={routed.tolist()} K={[int(layer.K[e]) for e in routed]}")
    xt, xd = synth.moe_token_inputs(0)
    gu = [dev_linear(layer.gate[e]) for e in routed] + [dev_linear(layer.up[e]) for e in routed]
    t_gu = tb.ExpertTable(gu, shared_side=0)
    y_gu = tb.trellis_moe_gemv(t_gu, to_dev(np.arange(16, dtype=np.int32)), to_dev(xt[0]), False,
                               to_dev(layer.r_hidden_in), to_dev(layer.s_hidden_in), 0)
    t_d = tb.ExpertTable([dev_linear(layer.down[e]) for e in routed], shared_side=1)
    y_d = tb.trellis_moe_gemv(t_d, to_dev(np.arange(8, dtype=np.int32)), to_dev(xd), True,
                              to_dev(layer.r_hidden_out), to_dev(layer.s_hidden_out), 1)
    torch.cuda.synchronize()
    g_ref, u_ref, d_ref = O.moe_forward(layer, routed, xt, xd)
    y_gu = y_gu.cpu().numpy().astype(np.float64)
    assert rel_l2(y_gu[:8], g_ref) < REL_L2_TOL
    assert rel_l2(y_gu[8:], u_ref) < REL_L2_TOL
    assert rel_l2(y_d.cpu().numpy(), d_ref) < REL_L2_TOL
    for k in range(8):  # and each expert's rows on their own
        assert rel_l2(y_gu[k], g_ref[k]) < REL_L2_TOL and rel_l2(y_gu[8 + k], u_ref[k]) < REL_L2_TOL


# ------------------------------------------------------------------------------------------
# One workspace for every entry point
# ------------------------------------------------------------------------------------------

def test_one_workspace_serves_every_entry_point():
    """A zero-filled buffer sized for the largest request serves trellis_gemm, then
    trellis_gemv, trellis_moe_gemv, trellis_gemm_fp8 and trellis_gemv_list, in that order:
    the prefill products keep their scratch after the reserved region, so the small-batch
    counters stay zero and the error word untouched."""
    lin = synth.make_linear(np.random.SeedSequence(90), 3, 512, 384)
    lin8 = synth.make_linear(np.random.SeedSequence(91), 2, 512, 384)
    lin8.cb = 2
    L, L8 = dev_linear(lin), dev_linear(lin8)
    xm = synth.make_x(np.random.SeedSequence(92), 300, 512)
    xb = synth.make_x(np.random.SeedSequence(93), 2, 512)
    table = tb.ExpertTable([L, L8])
    nb = max(L.workspace_bytes(tb.TRELLIS_OP_GEMM, 300), L8.workspace_bytes(tb.TRELLIS_OP_GEMM_FP8, 300),
             L.workspace_bytes(tb.TRELLIS_OP_GEMV, 2), table.workspace_bytes(2),
             tb.trellis_gemv_list_workspace_bytes([L, L8], 2))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    ym = tb.trellis_gemm(L, to_dev(xm), ws=ws).cpu().numpy()
    assert _counters_zero(ws)
    yv = tb.trellis_gemv(L, to_dev(xb), ws=ws).cpu().numpy()
    ye = tb.trellis_moe_gemv(table, to_dev(np.array([1, 0], np.int32)), to_dev(xb[0]), False, ws=ws).cpu().numpy()
    y8 = tb.trellis_gemm_fp8(L8, to_dev(xm), ws=ws).cpu().numpy()
    yl = [y.cpu().numpy() for y in tb.trellis_gemv_list([L, L8], [to_dev(xb), to_dev(xb)], ws=ws)]
    torch.cuda.synchronize()
    assert rel_l2(ym, O.forward_linear(lin, xm)) < REL_L2_TOL
    assert rel_l2(yv, O.forward_linear(lin, xb)) < REL_L2_TOL
    assert rel_l2(ye[0], O.forward_linear(lin8, xb[:1])[0]) < REL_L2_TOL
    assert rel_l2(ye[1], O.forward_linear(lin, xb[:1])[0]) < REL_L2_TOL
    assert rel_l2(y8, O.forward_linear(lin8, xm, act_e4m3=True)) < REL_L2_TOL
    assert rel_l2(yl[0], O.forward_linear(lin, xb)) < REL_L2_TOL
    assert rel_l2(yl[1], O.forward_linear(lin8, xb)) < REL_L2_TOL
    assert _counters_zero(ws) and tb.error_word(ws) == 0
