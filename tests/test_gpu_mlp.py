"""GPU parity: trellis_moe_mlp (the fused routed-expert MLP) against the fp64 CPU oracle.

y and the activations a = silu(gate x) * up x must be within 2e-3 relative L2 of the
oracle.  At the GLM-like full size the oracle computes the whole token (all eight routed
experts: every activation and every output channel); the eight-expert call is also checked
through linearity in the router weights."""
import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb
from trellis_coded_bit_amd import synth

from gpu_util import REL_L2_TOL, log_case, rel_l2, to_dev

pytestmark = pytest.mark.gpu


def _run(tables, routed, w, x, ws=None, want_act=True):
    n = len(routed)
    act = torch.empty((n, tables.inter), dtype=torch.float16, device="cuda") if want_act else None
    y = tb.trellis_moe_mlp(tables, to_dev(np.asarray(routed, np.int32)), to_dev(np.asarray(w, np.float32)),
                           to_dev(np.ascontiguousarray(x).reshape(-1)), tables.r_hidden_in, tables.s_hidden_in,
                           tables.r_hidden_out, tables.s_hidden_out, act=act, ws=ws)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    return (y, act.cpu().numpy().astype(np.float64)) if want_act else y


def _small(halves, seed=0):
    return synth.moe_mlp_layer(seed, n_experts=6, hidden=384, inter=512, halves=halves)


@pytest.mark.parametrize("halves", [1, 2, 4])
def test_mlp_small(halves):
    log_case(f"mlp small halves={halves}")
    layer = _small(halves)
    tables = tb.MoEMLPTables.from_host(layer)
    routed = [5, 0, 3, 3, 1]
    w = synth.moe_router_weights(halves, 1, len(routed))[0]
    x = synth.make_x(np.random.SeedSequence(21), 1, 384)
    ws = torch.zeros(tables.workspace_bytes(len(routed)), dtype=torch.uint8, device="cuda")
    y, act = _run(tables, routed, w, x, ws)
    y_ref, a_ref = O.moe_mlp_forward(layer, routed, w, x, return_act=True)
    assert rel_l2(y, y_ref) < REL_L2_TOL
    for k in range(len(routed)):
        assert rel_l2(act[k], a_ref[k]) < REL_L2_TOL, k
    assert int(ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("wgs", ["7", "13", "64"])
def test_mlp_ranges_spanning_problems(monkeypatch, wgs):
    """Few workgroups: ranges cross slice, expert and column-block boundaries."""
    log_case(f"mlp wgs={wgs}")
    monkeypatch.setenv("TRELLIS_GEMV_WGS", wgs)
    layer = _small(4, seed=1)
    tables = tb.MoEMLPTables.from_host(layer)
    routed = [2, 4, 1]
    w = [0.5, -0.25, 1.5]
    x = synth.make_x(np.random.SeedSequence(22), 1, 384)
    y, act = _run(tables, routed, w, x)
    y_ref, a_ref = O.moe_mlp_forward(layer, routed, w, x, return_act=True)
    assert rel_l2(y, y_ref) < REL_L2_TOL
    assert rel_l2(act, a_ref) < REL_L2_TOL


def test_mlp_no_routed_experts_writes_zeros():
    layer = _small(2)
    tables = tb.MoEMLPTables.from_host(layer)
    y = torch.full((384,), 3.0, dtype=torch.float16, device="cuda")
    tb.trellis_moe_mlp(tables, torch.empty(0, dtype=torch.int32, device="cuda"),
                       torch.empty(0, dtype=torch.float32, device="cuda"),
                       to_dev(synth.make_x(np.random.SeedSequence(1), 1, 384)[0]), tables.r_hidden_in,
                       tables.s_hidden_in, tables.r_hidden_out, tables.s_hidden_out, out=y)
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def test_mlp_bad_routed_id_contributes_zero_and_sets_error_word():
    layer = _small(2, seed=2)
    tables = tb.MoEMLPTables.from_host(layer)
    routed = [1, 9, 4, -1]  # 9 and -1 are out of range
    w = [0.4, 0.3, 0.6, 0.2]
    x = synth.make_x(np.random.SeedSequence(23), 1, 384)
    ws = torch.zeros(tables.workspace_bytes(len(routed)), dtype=torch.uint8, device="cuda")
    y, act = _run(tables, routed, w, x, ws)
    y_ref, a_ref = O.moe_mlp_forward(layer, [1, 4], [0.4, 0.6], x, return_act=True)
    assert rel_l2(y, y_ref) < REL_L2_TOL
    assert np.all(act[1] == 0) and np.all(act[3] == 0)
    assert rel_l2(act[[0, 2]], a_ref) < REL_L2_TOL
    assert int(ws[:4].view(torch.int32).item()) != 0


def test_mlp_deterministic_and_shape_changes_share_workspace():
    layer = _small(4, seed=3)
    tables = tb.MoEMLPTables.from_host(layer)
    x = synth.make_x(np.random.SeedSequence(24), 1, 384)
    ws = torch.zeros(tables.workspace_bytes(6), dtype=torch.uint8, device="cuda")
    r8, w8 = [0, 1, 2, 3, 4, 5], [0.1, 0.2, 0.1, 0.3, 0.2, 0.1]
    y1 = _run(tables, r8, w8, x, ws, want_act=False)
    y_small = _run(tables, [3], [1.0], x, ws, want_act=False)
    y2 = _run(tables, r8, w8, x, ws, want_act=False)
    assert np.array_equal(y1, y2)
    assert rel_l2(y_small, O.moe_mlp_forward(layer, [3], [1.0], x)) < REL_L2_TOL


def test_mlp_glm_like_full_size():
    """8 of 256 GLM-like experts (hidden 6144, intermediate 2048, 16 gate/up halves per
    expert with per-half widths, down one width per expert), the launch configuration the
    benchmark times (the grid depends on n and the shapes, not on the table length)."""
    import dataclasses
    routed = synth.moe_routes(0, 1)[0]
    full = synth.moe_mlp_layer(0, experts=routed.tolist())
    layer = dataclasses.replace(full, gate=[full.gate[e] for e in routed], up=[full.up[e] for e in routed],
                                down=[full.down[e] for e in routed], K_gu=full.K_gu[routed], K_d=full.K_d[routed])
    log_case(f"mlp full routed={routed.tolist()} K_d={layer.K_d.tolist()}")
    tables = tb.MoEMLPTables.from_host(layer)
    idx = np.arange(8, dtype=np.int32)
    w = synth.moe_router_weights(0, 1)[0]
    x = synth.make_x(np.random.SeedSequence(25), 1, 6144)
    y, act = _run(tables, idx, w, x)

    # linearity in the router weights: the eight-expert call against eight one-expert calls
    singles = [_run(tables, [int(k)], [1.0], x, want_act=False) for k in idx]
    assert rel_l2(y, sum(float(w[k]) * singles[k] for k in range(8))) < REL_L2_TOL
    # the whole token through the oracle: every expert's activations, every output channel
    ref_y, ref_act = O.moe_mlp_forward(layer, idx, w, x, return_act=True)
    assert rel_l2(y, ref_y) < REL_L2_TOL
    for k in range(8):
        assert rel_l2(act[k], ref_act[k]) < REL_L2_TOL, k
        for h in range(16):  # no 128-channel half off on its own
            assert rel_l2(act[k, 128 * h:128 * h + 128], ref_act[k, 128 * h:128 * h + 128]) < REL_L2_TOL, (k, h)
    for J in range(6144 // 128):
        assert rel_l2(y[128 * J:128 * J + 128], ref_y[128 * J:128 * J + 128]) < REL_L2_TOL, J
