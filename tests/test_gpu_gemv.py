"""GPU parity: trellis_gemv and trellis_moe_gemv against the fp64 CPU oracle.

Outputs must be within 2e-3 relative L2 of the oracle.  Full-size workloads are checked on
sampled 128-column output blocks (which the oracle computes from those blocks' tiles only)."""
import os

import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, dev_linear, log_case, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _gemv_np(lin, x):
    y = tb.trellis_gemv(dev_linear(lin), to_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def test_gemv_single_k2_workload():
    wl = synth.single_k2(0)
    lin, x = wl.layers["w"], wl.xs["w"]
    y = _gemv_np(lin, x)
    ref = O.forward_linear(lin, x)
    assert rel_l2(y, ref) < REL_L2_TOL


@pytest.mark.parametrize("K", [2, 3, 4])
@pytest.mark.parametrize("n_in,n_out,B", [(384, 640, 1), (1152, 256, 3), (128, 128, 8), (640, 384, 5)])
def test_gemv_small_shapes(K, n_in, n_out, B):
    log_case(f"gemv K={K} {n_in}x{n_out} B={B}")
    lin = synth.make_linear(np.random.SeedSequence([K, n_in, n_out, B]), K, n_in, n_out)
    x = synth.make_x(np.random.SeedSequence([B, 1]), B, n_in)
    y = _gemv_np(lin, x)
    ref = O.forward_linear(lin, x)
    assert y.shape == ref.shape
    assert rel_l2(y, ref) < REL_L2_TOL
    # every batch row separately too
    for b in range(B):
        assert rel_l2(y[b], ref[b]) < REL_L2_TOL


@pytest.mark.parametrize("wgs", ["3", "7", "1"])
def test_gemv_ranges_spanning_column_blocks(monkeypatch, wgs):
    """Few workgroups: each range covers several column blocks and cuts them mid-way, so the
    partial-sum fixup and the counters are exercised."""
    monkeypatch.setenv("TRELLIS_GEMV_WGS", wgs)
    log_case(f"gemv spanning wgs={wgs}")
    lin = synth.make_linear(np.random.SeedSequence(5), 3, 640, 896)
    x = synth.make_x(np.random.SeedSequence(6), 2, 640)
    y = _gemv_np(lin, x)
    assert rel_l2(y, O.forward_linear(lin, x)) < REL_L2_TOL


def test_gemv_back_to_back_deterministic():
    """Repeated calls reuse the workspace (counters self-reset) and give identical bits."""
    lin = synth.make_linear(np.random.SeedSequence(8), 2, 1024, 768)
    x = to_dev(synth.make_x(np.random.SeedSequence(9), 4, 1024))
    L = dev_linear(lin)
    ys = [tb.trellis_gemv(L, x).clone() for _ in range(4)]
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    ref = O.forward_linear(lin, x.cpu().numpy())
    assert rel_l2(ys[-1].cpu().numpy(), ref) < REL_L2_TOL


@pytest.mark.parametrize("which", ["gate", "up", "down"])
def test_gemv_dense_mlp_full_size(which):
    log_case(f"gemv dense MLP {which}")
    wl = synth.dense_mlp(0)
    lin, x = wl.layers[which], wl.xs[which]
    y = _gemv_np(lin, x)
    nJ = lin.out_features // 128
    blocks = sorted({0, nJ - 1, *np.random.default_rng(2).integers(0, nJ, 2).tolist()})
    ref = O.forward_linear(lin, x, col_blocks=blocks)
    got = np.concatenate([y[:, 128 * J:128 * J + 128] for J in blocks], axis=1)
    assert rel_l2(got, ref) < REL_L2_TOL


def test_dense_mlp_gate_up_as_one_launch():
    """The dense step's gate (K2) and up (K3) share x and run as one launch over a 2-entry
    table: each output row must match the oracle (sampled column blocks)."""
    log_case("gate+up one launch")
    wl = synth.dense_mlp(0)
    gate, up, x = wl.layers["gate"], wl.layers["up"], wl.xs["gate"]
    table = tb.ExpertTable([dev_linear(gate), dev_linear(up)])
    routed = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    y = tb.trellis_moe_gemv(table, routed, to_dev(x[0]), False).cpu().numpy()
    blocks = [0, 77, 135]
    for row, lin in enumerate([gate, up]):
        ref = O.forward_linear(lin, x, col_blocks=blocks)
        got = np.concatenate([y[row:row + 1, 128 * J:128 * J + 128] for J in blocks], axis=1)
        assert rel_l2(got, ref) < REL_L2_TOL, row


def test_gemv_shape_changes_share_workspace():
    """Calls of different shapes back to back on one workspace (the counters of a wide call
    must not be disturbed by the partial sums of an earlier narrow one)."""
    shapes = [(17408, 5120), (5120, 10240), (1024, 384), (5120, 17408), (2048, 6144)]
    for i, (n_in, n_out) in enumerate(shapes):
        lin = synth.make_linear(np.random.SeedSequence([60, i]), 2, n_in, n_out)
        x = synth.make_x(np.random.SeedSequence([61, i]), 1, n_in)
        y = _gemv_np(lin, x)
        nJ = n_out // 128
        blocks = sorted({0, nJ - 1})
        ref = O.forward_linear(lin, x, col_blocks=blocks)
        got = np.concatenate([y[:, 128 * J:128 * J + 128] for J in blocks], axis=1)
        assert rel_l2(got, ref) < REL_L2_TOL, (n_in, n_out)


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_gemv_small_batch_full_size(B):
    log_case(f"gemv small-batch B={B}")
    wl = synth.small_batch(0, batch=B)
    for name in ("qkv", "z", "out"):
        lin, x = wl.layers[name], wl.xs[name]
        y = _gemv_np(lin, x)
        nJ = lin.out_features // 128
        blocks = sorted({0, nJ - 1, int(np.random.default_rng(B).integers(0, nJ))})
        ref = O.forward_linear(lin, x, col_blocks=blocks)
        got = np.concatenate([y[:, 128 * J:128 * J + 128] for J in blocks], axis=1)
        assert rel_l2(got, ref) < REL_L2_TOL, name


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
    assert int(ws[:4].view(torch.int32).item()) == 0


def test_moe_bad_entries_give_zero_rows_and_error_word():
    lins, sr, ss = _moe_small(-1)
    devl = [dev_linear(l) for l in lins[:3]]
    table = tb.ExpertTable(devl)
    # corrupt entry 1's K on the device copy (the kernel must reject it, not decode it)
    raw = bytearray(table.table.cpu().numpy().tobytes())
    sz = len(raw) // 3
    raw[sz + 40:sz + 44] = (9).to_bytes(4, "little")  # K field of entry 1
    table.table = torch.frombuffer(raw, dtype=torch.uint8).cuda()
    routed = to_dev(np.array([0, 1, 7, 2], np.int32))  # entry 1 bad K, id 7 out of range
    x = to_dev(synth.make_x(np.random.SeedSequence(3), 1, 256)[0])
    ws = torch.zeros(table.workspace_bytes(4), dtype=torch.uint8, device="cuda")
    y = tb.trellis_moe_gemv(table, routed, x, False, ws=ws)
    torch.cuda.synchronize()
    yn = y.cpu().numpy()
    assert np.all(yn[1] == 0) and np.all(yn[2] == 0)
    assert np.any(yn[0] != 0) and np.any(yn[3] != 0)
    assert int(ws[:4].view(torch.int32).item()) != 0


def test_moe_glm_like_full_size():
    """8 routed experts of the GLM-like layer (6144 <-> 2048, K per expert from 2/3/4):
    gate+up in one launch over a 16-entry table with the shared hidden-side input vectors,
    down with per-expert inputs and the shared hidden-side output vectors."""
    routed = synth.moe_routes(0, 1)[0]
    layer = synth.moe_layer(0, experts=routed.tolist())
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
    y_gu = y_gu.cpu().numpy().astype(np.float64)
    y_d = y_d.cpu().numpy().astype(np.float64)
    blocks_i = [0, 15]  # of the 2048-wide gate/up outputs
    blocks_h = [0, 47]  # of the 6144-wide down outputs
    g_ref, u_ref, d_ref = O.moe_forward(layer, routed, xt, xd, col_blocks=(blocks_i, blocks_h))
    pick = lambda y, bl: np.concatenate([y[:, 128 * J:128 * J + 128] for J in bl], axis=1)
    assert rel_l2(pick(y_gu[:8], blocks_i), g_ref) < REL_L2_TOL
    assert rel_l2(pick(y_gu[8:], blocks_i), u_ref) < REL_L2_TOL
    assert rel_l2(pick(y_d, blocks_h), d_ref) < REL_L2_TOL
