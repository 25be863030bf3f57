"""Seeded synthetic workloads for the trellis-coded linear layers.

This module only draws random numbers.  It holds none of the method's
arithmetic (no decode, no rotation, no scaling): both the GPU path and the CPU
oracle consume the host arrays it returns.

Distributions (one ``numpy.random.Generator(PCG64)`` child per tensor, spawned
in a fixed order from ``SeedSequence(seed)``):

* ``code``: uniform 16-bit words, shape [in/16, out/16, 16*K] (int16).  Every
  circular bitstring is a valid tail-biting trellis path, so uniform words are
  legal codes; real codes also look uniform when read as independent words
  (escha FORMAT page, "Bit layout").
* ``rin`` / ``rout``: fp16 drawn from U[0.5, 1.5].
* ``s_in`` / ``s_out``: f32 drawn from N(1, 0.02) (std 0.02), or exactly 1.0.
* ``x``: fp16 drawn from N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

HIDDEN_MOE = 6144
INTER_MOE = 2048
N_EXPERTS = 256
N_ROUTED = 8
MOE_K_CHOICES = (2, 3, 4)
MOE_K_PROBS = (0.3, 0.5, 0.2)


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


@dataclasses.dataclass
class Linear:
    """Host arrays of one trellis-coded linear layer y = x @ W, W [in, out]."""

    K: int
    in_features: int
    out_features: int
    code: np.ndarray  # int16 [in/16, out/16, 16*K]
    rin: np.ndarray  # float16 [in]
    rout: np.ndarray  # float16 [out]
    s_in: np.ndarray  # float32 [in]
    s_out: np.ndarray  # float32 [out]
    cb: int = 1  # codebook: 1 = MCG fp16 values, 2 = the same rounded to E4M3

    @property
    def code_bytes(self) -> int:
        return self.in_features * self.out_features * self.K // 8


def make_linear(seed_seq: np.random.SeedSequence, K: int, in_features: int, out_features: int,
                unit_s: bool = False, code_only_seed: bool = False) -> Linear:
    """Draw one layer.  Children are spawned in the order code, rin, rout, s_in, s_out."""
    assert in_features % 16 == 0 and out_features % 16 == 0
    c_code, c_rin, c_rout, c_sin, c_sout = seed_seq.spawn(5)
    code = _rng(c_code).integers(0, 1 << 16, size=(in_features // 16, out_features // 16, 16 * K),
                                 dtype=np.uint16).view(np.int16)
    rin = _rng(c_rin).uniform(0.5, 1.5, size=in_features).astype(np.float16)
    rout = _rng(c_rout).uniform(0.5, 1.5, size=out_features).astype(np.float16)
    if unit_s:
        s_in = np.ones(in_features, np.float32)
        s_out = np.ones(out_features, np.float32)
    else:
        s_in = _rng(c_sin).normal(1.0, 0.02, size=in_features).astype(np.float32)
        s_out = _rng(c_sout).normal(1.0, 0.02, size=out_features).astype(np.float32)
    return Linear(K, in_features, out_features, code, rin, rout, s_in, s_out)


def make_x(seed_seq: np.random.SeedSequence, rows: int, n: int) -> np.ndarray:
    return _rng(seed_seq).normal(0.0, 1.0, size=(rows, n)).astype(np.float16)


# --------------------------------------------------------------------------------------
# The five workloads.  Shapes come from the 27B dense layer shapes (hidden 5120, MLP 17408,
# in_proj_qkv 10240x5120, in_proj_z 6144x5120, out_proj 5120x6144) and the GLM-like MoE
# experts (hidden 6144, inner 2048, 256 experts, 8 routed).
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    layers: Dict[str, Linear]
    xs: Dict[str, np.ndarray]  # per layer name: fp16 [rows, in]


def single_k2(seed: int = 0) -> Workload:
    """K=2, 512 -> 256, s = 1.0 exactly, batch 1."""
    root = np.random.SeedSequence(seed)
    c_lin, c_x = root.spawn(2)
    lin = make_linear(c_lin, 2, 512, 256, unit_s=True)
    return Workload("single K2 512x256", {"w": lin}, {"w": make_x(c_x, 1, 512)})


def dense_mlp(seed: int = 0, batch: int = 1) -> Workload:
    """gate K2 5120->17408, up K3 5120->17408, down K3 17408->5120, batch 1."""
    root = np.random.SeedSequence(seed)
    cg, cu, cd, cxg, cxd = root.spawn(5)
    layers = {
        "gate": make_linear(cg, 2, 5120, 17408),
        "up": make_linear(cu, 3, 5120, 17408),
        "down": make_linear(cd, 3, 17408, 5120),
    }
    xg = make_x(cxg, batch, 5120)
    xd = make_x(cxd, batch, 17408)
    return Workload("dense MLP decode 5120<->17408 (K2 gate, K3 up/down)", layers,
                    {"gate": xg, "up": xg, "down": xd})


def small_batch(seed: int = 0, batch: int = 1) -> Workload:
    """qkv K2 5120->10240, z K2 5120->6144, out K2 6144->5120 at batch 1/2/4/8."""
    root = np.random.SeedSequence(seed)
    cq, cz, co, cx, cxo = root.spawn(5)
    layers = {
        "qkv": make_linear(cq, 2, 5120, 10240),
        "z": make_linear(cz, 2, 5120, 6144),
        "out": make_linear(co, 2, 6144, 5120),
    }
    x = make_x(cx, batch, 5120)
    xo = make_x(cxo, batch, 6144)
    return Workload(f"small-batch decode K2 (qkv 5120x10240, z 5120x6144, out 6144x5120) B={batch}",
                    layers, {"qkv": x, "z": x, "out": xo})


def prefill(seed: int = 0, M: int = 2048) -> Workload:
    """K3 5120->17408 with M tokens."""
    root = np.random.SeedSequence(seed)
    cl, cx = root.spawn(2)
    lin = make_linear(cl, 3, 5120, 17408)
    return Workload(f"prefill K3 5120x17408 M={M}", {"w": lin}, {"w": make_x(cx, M, 5120)})


@dataclasses.dataclass
class MoELayer:
    """256 experts; gate/up [6144 -> 2048], down [2048 -> 6144].

    The hidden-side vectors (6144 wide) are one per layer and shared by every expert:
    ``r_hidden_in``/``s_hidden_in`` scale the gate/up inputs and ``r_hidden_out``/
    ``s_hidden_out`` scale the down outputs.  The 2048-wide side keeps per-expert vectors
    (the ``rout``/``s_out`` of gate/up and the ``rin``/``s_in`` of down).  The hidden-side
    fields of the per-expert ``Linear`` objects are left as drawn but are not used.
    """

    K: np.ndarray  # int32 [E]
    gate: List[Linear]
    up: List[Linear]
    down: List[Linear]
    r_hidden_in: np.ndarray
    s_hidden_in: np.ndarray
    r_hidden_out: np.ndarray
    s_hidden_out: np.ndarray

    def expert_code_bytes(self, e: int) -> int:
        return self.gate[e].code_bytes + self.up[e].code_bytes + self.down[e].code_bytes


def moe_layer(seed: int = 0, n_experts: int = N_EXPERTS, hidden: int = HIDDEN_MOE,
              inner: int = INTER_MOE, experts: Optional[List[int]] = None) -> MoELayer:
    """Draw the MoE layer.  ``experts`` limits which experts get code arrays (others None);
    the per-expert children are spawned for all experts so any subset is reproducible."""
    root = np.random.SeedSequence(seed)
    c_k, c_hid, c_exp = root.spawn(3)
    K = _rng(c_k).choice(np.array(MOE_K_CHOICES, np.int32), size=n_experts, p=MOE_K_PROBS)
    ch = c_hid.spawn(4)
    r_hi = _rng(ch[0]).uniform(0.5, 1.5, size=hidden).astype(np.float16)
    s_hi = _rng(ch[1]).normal(1.0, 0.02, size=hidden).astype(np.float32)
    r_ho = _rng(ch[2]).uniform(0.5, 1.5, size=hidden).astype(np.float16)
    s_ho = _rng(ch[3]).normal(1.0, 0.02, size=hidden).astype(np.float32)
    per = c_exp.spawn(n_experts)
    gate, up, down = [None] * n_experts, [None] * n_experts, [None] * n_experts
    for e in (range(n_experts) if experts is None else experts):
        cg, cu, cd = per[e].spawn(3)
        k = int(K[e])
        gate[e] = make_linear(cg, k, hidden, inner)
        up[e] = make_linear(cu, k, hidden, inner)
        down[e] = make_linear(cd, k, inner, hidden)
    return MoELayer(K, gate, up, down, r_hi, s_hi, r_ho, s_ho)


def moe_routes(seed: int, n_tokens: int, n_experts: int = N_EXPERTS, n_routed: int = N_ROUTED) -> np.ndarray:
    """int32 [n_tokens, n_routed]: distinct expert ids per token, uniform without replacement."""
    rng = _rng(np.random.SeedSequence([seed, 0x524F55]))
    return np.stack([rng.choice(n_experts, size=n_routed, replace=False) for _ in range(n_tokens)]).astype(np.int32)


def moe_token_inputs(seed: int, hidden: int = HIDDEN_MOE, inner: int = INTER_MOE, n_routed: int = N_ROUTED):
    """Token activation x [1, hidden] for gate/up and per-expert down inputs [n_routed, inner]."""
    cx, cd = np.random.SeedSequence([seed, 0x544F4B]).spawn(2)
    return make_x(cx, 1, hidden), make_x(cd, n_routed, inner)


# --------------------------------------------------------------------------------------
# Routed-expert MLP with per-half widths (EXLR8 page: a "half" is 128 of an expert's
# intermediate channels and the storage unit of gate/up; down has one width per expert).
# --------------------------------------------------------------------------------------

HALF = 128


@dataclasses.dataclass
class MoEMLPLayer:
    """E experts; gate/up stored as ``halves`` column slices [hidden -> inter/halves] each
    with its own width, down [inter -> hidden] with one width per expert.

    The hidden-side vectors are shared by every expert (one per layer); the per-half
    ``Linear`` objects carry references to the shared input-side arrays (no copies) and
    their own output-side vectors for their channels.  Down's output-side fields are the
    shared ``r_hidden_out``/``s_hidden_out`` references.
    """

    hidden: int
    inter: int
    halves: int
    K_gu: np.ndarray  # int32 [E, halves]: width of half h of expert e (gate and up alike)
    K_d: np.ndarray  # int32 [E]
    gate: List[Optional[List[Linear]]]  # [E][halves]
    up: List[Optional[List[Linear]]]
    down: List[Optional[Linear]]
    r_hidden_in: np.ndarray
    s_hidden_in: np.ndarray
    r_hidden_out: np.ndarray
    s_hidden_out: np.ndarray

    def expert_code_bytes(self, e: int) -> int:
        return (sum(l.code_bytes for l in self.gate[e]) + sum(l.code_bytes for l in self.up[e])
                + self.down[e].code_bytes)


def _half_linear(ss: np.random.SeedSequence, K: int, hidden: int, width: int, r_in, s_in) -> Linear:
    """One gate/up half: children spawned in the order code, rout, s_out.  s_out is drawn
    from N(1, 0.02) / sqrt(hidden): the projection's global scale (the EXLR8 page folds one
    per projection into the stored side vectors) keeps outputs of order one."""
    c_code, c_rout, c_sout = ss.spawn(3)
    code = _rng(c_code).integers(0, 1 << 16, size=(hidden // 16, width // 16, 16 * K),
                                 dtype=np.uint16).view(np.int16)
    rout = _rng(c_rout).uniform(0.5, 1.5, size=width).astype(np.float16)
    s_out = (_rng(c_sout).normal(1.0, 0.02, size=width) / np.sqrt(hidden)).astype(np.float32)
    return Linear(K, hidden, width, code, r_in, rout, s_in, s_out)


def _down_linear(ss: np.random.SeedSequence, K: int, inter: int, hidden: int, r_out, s_out) -> Linear:
    """Down of one expert: children spawned in the order code, rin, s_in; s_in is drawn from
    N(1, 0.02) / sqrt(inter) (the global scale, as for gate/up)."""
    c_code, c_rin, c_sin = ss.spawn(3)
    code = _rng(c_code).integers(0, 1 << 16, size=(inter // 16, hidden // 16, 16 * K),
                                 dtype=np.uint16).view(np.int16)
    rin = _rng(c_rin).uniform(0.5, 1.5, size=inter).astype(np.float16)
    s_in = (_rng(c_sin).normal(1.0, 0.02, size=inter) / np.sqrt(inter)).astype(np.float32)
    return Linear(K, inter, hidden, code, rin, r_out, s_in, s_out)


def moe_mlp_layer(seed: int = 0, n_experts: int = N_EXPERTS, hidden: int = HIDDEN_MOE,
                  inter: int = INTER_MOE, halves: int = INTER_MOE // HALF,
                  experts: Optional[List[int]] = None) -> MoEMLPLayer:
    """Draw a routed-expert MLP layer.  Widths: K ~ choice({2,3,4}, p = .3/.5/.2) per
    (expert, half) for gate/up and per expert for down.  ``experts`` limits which experts
    get arrays (the children of every expert are spawned, so any subset is reproducible)."""
    assert inter % (halves * 16) == 0
    width = inter // halves
    root = np.random.SeedSequence([seed, 0x4D4C50])
    c_kgu, c_kd, c_hid, c_exp = root.spawn(4)
    K_gu = _rng(c_kgu).choice(np.array(MOE_K_CHOICES, np.int32), size=(n_experts, halves), p=MOE_K_PROBS)
    K_d = _rng(c_kd).choice(np.array(MOE_K_CHOICES, np.int32), size=n_experts, p=MOE_K_PROBS)
    ch = c_hid.spawn(4)
    r_hi = _rng(ch[0]).uniform(0.5, 1.5, size=hidden).astype(np.float16)
    s_hi = _rng(ch[1]).normal(1.0, 0.02, size=hidden).astype(np.float32)
    r_ho = _rng(ch[2]).uniform(0.5, 1.5, size=hidden).astype(np.float16)
    s_ho = _rng(ch[3]).normal(1.0, 0.02, size=hidden).astype(np.float32)
    per = c_exp.spawn(n_experts)
    gate, up, down = [None] * n_experts, [None] * n_experts, [None] * n_experts
    for e in (range(n_experts) if experts is None else experts):
        cg, cu, cd = per[e].spawn(3)
        gate[e] = [_half_linear(c, int(K_gu[e, h]), hidden, width, r_hi, s_hi) for h, c in enumerate(cg.spawn(halves))]
        up[e] = [_half_linear(c, int(K_gu[e, h]), hidden, width, r_hi, s_hi) for h, c in enumerate(cu.spawn(halves))]
        down[e] = _down_linear(cd, int(K_d[e]), inter, hidden, r_ho, s_ho)
    return MoEMLPLayer(hidden, inter, halves, K_gu, K_d, gate, up, down, r_hi, s_hi, r_ho, s_ho)


def moe_router_weights(seed: int, n_tokens: int, n_routed: int = N_ROUTED) -> np.ndarray:
    """f32 [n_tokens, n_routed]: positive router weights summing to one per token
    (a flat Dirichlet draw)."""
    rng = _rng(np.random.SeedSequence([seed, 0x525754]))
    return rng.dirichlet(np.ones(n_routed), size=n_tokens).astype(np.float32)
