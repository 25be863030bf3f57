"""Plain CPU oracle for EXL3-style trellis-coded weights.  TEST INFRASTRUCTURE ONLY.

Sources (cited by page title and section; no line numbers):

* [ESCHA]  "The escha W2 format, recovered and verified" -- sections "Tensor mapping",
  "Reconstruction", "Codebook: cb=1 (MCG), verified", "Bit layout: the part that is easy
  to get wrong", "How each claim was verified".
* [METAL]  "Escha-W2 runs on Metal" (escha-mlx-evidence page) -- the tensor list, the
  reconstruction / activation-side paragraph, "Codebook 1 decode, three instructions",
  the tile / tensor-core permutation paragraph and the Shannon-bound paragraph.
* [EXLR8]  the EXLR8 format page -- the rotation paragraphs (Q = signs x Hadamard), the
  tile-coding paragraph (Viterbi over a 16-bit-state trellis), the shared hidden-side
  rotation paragraph, the calibration paragraph (the expert MLP's activation), the
  width-manifest paragraph (per-half widths) and the E4M3 paragraph (the FP8 codebook).

Readings taken where the pages are silent or disagree are named A1..A26 in the
docstrings and listed in the design notes.  Every function here follows the plain
definition; nothing is blocked, fused or reordered beyond what the definition states.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

# [ESCHA] "Codebook: cb=1 (MCG)" and [METAL] "Codebook 1 decode": the three constants.
MCG_MULT = 0xCBAC1FED
MCG_MASK = 0x8FFF8FFF
MCG_XOR = 0x3B603B60
# [ESCHA] "How each claim was verified", item 3: EXL3's codebook_scale.
CODEBOOK_SCALE = 1.24371088
HAD_N = 128


# ----------------------------------------------------------------------------------------
# Bit layout
# ----------------------------------------------------------------------------------------

def tile_u32(words: np.ndarray) -> np.ndarray:
    """16*K int16 words -> 8*K uint32, u32[i] = w[2i] | w[2i+1] << 16.

    [ESCHA] "Bit layout": the decoder reads a tile as 32-bit words.  Reading A1: the pair
    order inside a 32-bit word is little-endian, as the EXLR8 page's "little-endian int16"
    storage implies.  Works on any leading shape.
    """
    w = np.asarray(words).view(np.uint16).astype(np.uint32)
    return w[..., 0::2] | (w[..., 1::2] << np.uint32(16))


def stream_bits(words: np.ndarray) -> np.ndarray:
    """The tile bitstream: bit p = (u32[p >> 5] >> (31 - (p & 31))) & 1 (MSB-first per word).

    [ESCHA] "Bit layout": windows are taken from the 32-bit words with shifts that place
    earlier symbols at higher bit positions.  Returns uint8 [..., 256*K].
    """
    u = tile_u32(words)
    be = u.astype(">u4").view(np.uint8)  # each word's bytes, most significant first
    return np.unpackbits(be, axis=-1)


def _window_index(K: int) -> np.ndarray:
    """idx[s, k] = (s*K + K - 16 + k) mod 256K: the 16 stream bits of symbol s's state."""
    n = 256 * K
    s = np.arange(256)[:, None]
    k = np.arange(16)[None, :]
    return (s * K + K - 16 + k) % n


def tile_states(words: np.ndarray, K: int, chunk: int = 4096) -> np.ndarray:
    """16-bit trellis state of every symbol: uint16 [..., 256].

    state_s = the 16 stream bits that END with symbol s's own K bits, most significant
    first, wrapping circularly around the tile (tail-biting).

    [ESCHA] "Bit layout": symbol t+j of a lane uses the window at shift 14-2j of a 64-bit
    funnel of (previous word, current word), i.e. the window whose lowest K bits are the
    symbol's own bits; consecutive states overlap by 16-K bits.  [METAL] (tile paragraph)
    states the same window "at bit offset i*K" -- reading A2: the two differ by a constant
    index shift, and the [ESCHA] formula is taken as normative.  Reading A3: K = 3 and 4
    use the same continuous 32-bit MSB-first stream (the pages give the formula at K=2 only).
    """
    words = np.asarray(words)
    assert words.shape[-1] == 16 * K, (words.shape, K)
    lead = words.shape[:-1]
    flat = words.reshape(-1, 16 * K)
    idx = _window_index(K)
    weights = (1 << (15 - np.arange(16))).astype(np.uint32)
    out = np.empty((flat.shape[0], 256), np.uint16)
    for a in range(0, flat.shape[0], chunk):
        bits = stream_bits(flat[a:a + chunk])  # [c, 256K]
        win = bits[:, idx].astype(np.uint32)  # [c, 256, 16]
        out[a:a + chunk] = (win * weights).sum(axis=-1).astype(np.uint16)
    return out.reshape(lead + (256,))


# ----------------------------------------------------------------------------------------
# Codebook
# ----------------------------------------------------------------------------------------

def mcg_hash(states: np.ndarray) -> np.ndarray:
    """v = (state * 0xCBAC1FED) mod 2^32, then (v & 0x8FFF8FFF) ^ 0x3B603B60.

    [ESCHA] "Codebook: cb=1 (MCG)"; [METAL] "Codebook 1 decode".  Reading A5: the multiply
    wraps at 32 bits (both halves of the 32-bit word are used).  Returns uint32.
    """
    s = np.asarray(states).astype(np.uint64)
    v = (s * np.uint64(MCG_MULT)) & np.uint64(0xFFFFFFFF)
    v = (v & np.uint64(MCG_MASK)) ^ np.uint64(MCG_XOR)
    return v.astype(np.uint32)


def codebook(states: np.ndarray) -> np.ndarray:
    """fp16 codebook value: binary16(lo half) + binary16(hi half), rounded once to fp16.

    [ESCHA] "Codebook": value = fp16_lo(v) + fp16_hi(v).  Reading A4: the sum is rounded to
    binary16 (round to nearest even) because the format's codebook values are fp16 (EXLR8
    comparison table).  The float64 sum of two fp16 numbers is exact, so this is a single
    rounding of the exact sum.  Returns float16 of the same shape.
    """
    v = mcg_hash(states)
    lo = (v & np.uint32(0xFFFF)).astype(np.uint16).view(np.float16).astype(np.float64)
    hi = (v >> np.uint32(16)).astype(np.uint16).view(np.float16).astype(np.float64)
    return (lo + hi).astype(np.float16)


def codebook_table() -> np.ndarray:
    """All 65536 codebook values, float16."""
    return codebook(np.arange(1 << 16, dtype=np.uint32))


# ----------------------------------------------------------------------------------------
# E4M3 (the FP8 codebook variant)
# ----------------------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_magnitudes() -> np.ndarray:
    """Values of the codes 0..126 (sign bit clear), float64, increasing.

    OCP 8-bit floating point, E4M3 flavour: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent field 0 holds subnormals m/8 * 2^-6; code 0x7F is NaN and there are no
    infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    out = []
    for code in range(127):
        e, m = code >> 3, code & 7
        out.append((m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(out)


def e4m3_codes(v) -> np.ndarray:
    """Round to E4M3: nearest finite value, ties to the even code, saturating at +-448.
    Returns uint8 codes (sign in bit 7; a negative value that rounds to zero keeps its sign).

    [EXLR8] E4M3 paragraph: every codebook value is rounded to E4M3 with round-to-nearest-
    even and saturation.  Written out from the definition: the two neighbouring
    representable magnitudes are found and the nearer taken; on a tie the one whose code
    is even.  NaN inputs are outside the domain.
    """
    v = np.asarray(v, np.float64)
    mags = e4m3_magnitudes()
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)  # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def e4m3_value(codes) -> np.ndarray:
    """E4M3 codes (uint8, no NaN code) -> float64."""
    c = np.asarray(codes, np.uint8)
    mag = e4m3_magnitudes()[c & 0x7F]
    return np.where(c & 0x80, -mag, mag)


def e4m3_round(v) -> np.ndarray:
    return e4m3_value(e4m3_codes(v))


def codebook_e4m3(states: np.ndarray) -> np.ndarray:
    """E4M3 codebook code of each state (uint8): the fp16 codebook value rounded to E4M3.

    [EXLR8] E4M3 paragraph (decoding is EXL3's algorithm followed by the E4M3 rounding);
    reading A19: the rounding applies to the fp16 value codebook() produces.  Every
    codebook magnitude is below 3.96 (rounding to at most 4), so saturation never acts here.
    """
    return e4m3_codes(codebook(states).astype(np.float64))


# ----------------------------------------------------------------------------------------
# Tile permutation and placement
# ----------------------------------------------------------------------------------------

def symbol_position(s: np.ndarray):
    """Symbol index s (0..255) -> (row r, column c) inside the 16x16 tile.

    [METAL] tile paragraph, closed-form inverse: for output column c and lane pair
    (q, rh), t = 4*(4*(c&7) + q) + 2*((c>>3)&1) + rh, r = 8*rh + 2*q + {0,1}, e = r & 1.
    Reading A6: t counts element pairs, so s = 2t + e.  Reading A7: r is the input row
    (k) and c the output column (n) of W_inner[in, out].  Solving for (r, c):
    e = s&1, rh = (s>>1)&1, ch = (s>>2)&1, q = (s>>3)&3, c&7 = s>>5.
    """
    s = np.asarray(s)
    e = s & 1
    rh = (s >> 1) & 1
    ch = (s >> 2) & 1
    q = (s >> 3) & 3
    cl = s >> 5
    return 8 * rh + 2 * q + e, 8 * ch + cl


def tiles_to_matrix(values: np.ndarray) -> np.ndarray:
    """values [Ti, Tj, 256] (symbol order) -> matrix [16*Ti, 16*Tj].

    [ESCHA] "Bit layout": tile elements land by the forward permutation (tile[perm] =
    values, no transpose) and code[i, j] covers W_inner[16i:16i+16, 16j:16j+16], the
    input-tile index major.
    """
    Ti, Tj, n = values.shape
    assert n == 256
    r, c = symbol_position(np.arange(256))
    tiles = np.empty((Ti, Tj, 16, 16), values.dtype)
    tiles[:, :, r, c] = values
    return tiles.transpose(0, 2, 1, 3).reshape(16 * Ti, 16 * Tj)


def decode_tiles(code: np.ndarray, K: int, cb: int = 1) -> np.ndarray:
    """Packed code int16 [in/16, out/16, 16K] -> W_hat float16 [in, out] (codebook domain).

    cb = 1: the MCG codebook's fp16 values; cb = 2: those values rounded to E4M3
    (codebook_e4m3), returned as float16 (every E4M3 value is exactly representable).
    """
    code = np.asarray(code)
    Ti, Tj, nw = code.shape
    assert nw == 16 * K and cb in (1, 2)
    st = tile_states(code, K)
    vals = codebook(st) if cb == 1 else e4m3_value(codebook_e4m3(st)).astype(np.float16)
    return tiles_to_matrix(vals)


def decode_tiles_e4m3(code: np.ndarray, K: int) -> np.ndarray:
    """Packed code -> E4M3 codes uint8 [in, out] of the cb = 2 weights."""
    code = np.asarray(code)
    return tiles_to_matrix(codebook_e4m3(tile_states(code, K)))


# ----------------------------------------------------------------------------------------
# Hadamard rotation and scales
# ----------------------------------------------------------------------------------------

def sylvester(n: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix: H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]]."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n
    return h


def hadamard128() -> np.ndarray:
    """H_128 / sqrt(128): symmetric, orthogonal, its own inverse.

    [ESCHA] "Reconstruction": had_l / had_r are the normalised Sylvester Hadamard of size
    128.  Reading A9: the 1/sqrt(128) normalisation applies on each side.
    """
    return sylvester(HAD_N) / math.sqrt(HAD_N)


def had_blocks(z: np.ndarray) -> np.ndarray:
    """Apply H_128/sqrt(128) to each consecutive 128-block of the last axis (float64).

    [METAL] reconstruction paragraph: had_blockwise(., -1).
    """
    z = np.asarray(z, np.float64)
    n = z.shape[-1]
    assert n % HAD_N == 0
    blocks = z.reshape(z.shape[:-1] + (n // HAD_N, HAD_N))
    return (blocks @ hadamard128()).reshape(z.shape)  # H is symmetric


def side_scale(r: np.ndarray, s: Optional[np.ndarray]) -> np.ndarray:
    """su = rin * s_in (or sv = rout * s_out), float64.

    [METAL] reconstruction paragraph: su = rin*s_in, sv = rout*s_out.  Reading A8: the
    escha s vectors are included (the [ESCHA] reconstruction omits them as not part of
    EXL3).  s = None means all ones.
    """
    out = np.asarray(r).astype(np.float64)
    if s is not None:
        out = out * np.asarray(s).astype(np.float64)
    return out


# ----------------------------------------------------------------------------------------
# Forward
# ----------------------------------------------------------------------------------------

def forward(code: np.ndarray, K: int, rin, rout, s_in, s_out, x: np.ndarray,
            col_blocks: Optional[Sequence[int]] = None, row_chunk: int = 64, cb: int = 1,
            act_e4m3: bool = False) -> np.ndarray:
    """y = had(had(x * su) @ W_hat) * sv, float64 [B, out] (or [B, 128*len(col_blocks)]).

    [METAL] reconstruction paragraph: xh = had_blockwise(x*su); y_pre = xh @ W_hat;
    y = had_blockwise(y_pre) * sv.  Reading A11: no bias.  W_hat is decoded in chunks of
    tile rows (memory only; the sum is the plain matrix product).  ``col_blocks`` restricts
    the output to the listed 128-column blocks, which needs only those blocks' tiles.
    ``cb`` selects the codebook (decode_tiles).

    act_e4m3 (the FP8 prefill of [EXLR8]: the E4M3 weights of cb = 2 feed FP8 matrix
    multiplies, so the rotated activations are E4M3 too).  Reading A25: each row of xh is
    quantised with its own scale sc = max|xh_row| / 448, q = e4m3_round(xh_row / sc)
    (round to nearest even, saturating), and y_pre_row = sc * (q @ W_hat); an all-zero row
    has q = 0.
    """
    code = np.asarray(code)
    Ti, Tj, _ = code.shape
    if col_blocks is None:
        cols = np.arange(Tj)
    else:
        cols = np.concatenate([np.arange(8 * J, 8 * J + 8) for J in col_blocks])
    sub = code[:, cols, :]
    chunks = (decode_tiles(sub[a:a + row_chunk], K, cb) for a in range(0, Ti, row_chunk))
    ch = np.concatenate([np.arange(16 * j, 16 * j + 16) for j in cols])
    return _forward_rows(chunks, 16 * Ti, rin, s_in, np.asarray(rout)[ch],
                         None if s_out is None else np.asarray(s_out)[ch], x, act_e4m3)


def _forward_rows(w_chunks, n_in, rin, s_in, rout, s_out, x, act_e4m3):
    """The forward of the reconstruction paragraph with W_hat given as consecutive blocks of
    rows (decoded fp16 values, a multiple of 128 rows each except the last)."""
    x = np.atleast_2d(np.asarray(x)).astype(np.float64)
    assert x.shape[1] == n_in
    su = side_scale(rin, s_in)
    sv = side_scale(rout, s_out)
    xh = had_blocks(x * su)
    sc = np.ones(x.shape[0])
    if act_e4m3:
        amax = np.max(np.abs(xh), axis=1)
        sc = amax / E4M3_MAX
        xh = np.where(amax[:, None] > 0, e4m3_round(xh / np.where(amax > 0, sc, 1.0)[:, None]), 0.0)
    y_pre, a = None, 0
    for w in w_chunks:
        w = np.asarray(w).astype(np.float64)
        part = xh[:, a:a + w.shape[0]] @ w
        y_pre = part if y_pre is None else y_pre + part
        a += w.shape[0]
    assert a == n_in
    y_pre *= sc[:, None]
    return had_blocks(y_pre) * sv


def forward_decoded(w_hat: np.ndarray, rin, rout, s_in, s_out, x: np.ndarray, row_chunk: int = 1024,
                    act_e4m3: bool = False) -> np.ndarray:
    """forward() with the matrix already decoded: w_hat fp16 [in, out] = decode_tiles(code),
    so that one decode serves several inputs.  Same definition, same float64 arithmetic
    (the product is taken over blocks of row_chunk input rows and the blocks summed)."""
    w_hat = np.asarray(w_hat)
    chunks = (w_hat[a:a + row_chunk] for a in range(0, w_hat.shape[0], row_chunk))
    return _forward_rows(chunks, w_hat.shape[0], rin, s_in, rout, s_out, x, act_e4m3)


def forward_linear(lin, x, col_blocks=None, act_e4m3: bool = False) -> np.ndarray:
    """forward() on a ``synth.Linear``-like object (its ``cb``, default 1)."""
    return forward(lin.code, lin.K, lin.rin, lin.rout, lin.s_in, lin.s_out, x, col_blocks,
                   cb=getattr(lin, "cb", 1), act_e4m3=act_e4m3)


def dense_weight(code: np.ndarray, K: int, rin, rout, s_in, s_out) -> np.ndarray:
    """Dense W [in, out] = diag(su) . Hblk . W_hat . Hblk . diag(sv), float64.

    [ESCHA] "Reconstruction": W = had_l(W_inner) * rin[:, None], then had_r(.) * rout[None, :]
    (with reading A8's s vectors folded into su / sv).  Used only to cross-check forward().
    """
    w = decode_tiles(code, K).astype(np.float64)
    n_in, n_out = w.shape
    hl = np.kron(np.eye(n_in // HAD_N), hadamard128())
    hr = np.kron(np.eye(n_out // HAD_N), hadamard128())
    return side_scale(rin, s_in)[:, None] * (hl @ w @ hr) * side_scale(rout, s_out)[None, :]


def moe_forward(layer, routed: Iterable[int], x_token: np.ndarray, x_down: np.ndarray,
                col_blocks=None):
    """Per routed expert e: gate/up outputs from the shared token x, down output from x_down[k].

    [EXLR8] shared-rotation paragraph: the hidden side (6144) of every expert uses one
    per-layer vector, so the token activation is rotated once and reused by every routed
    expert.  Reading A13: hidden-side scale vectors r_hidden_in/s_hidden_in (gate/up input)
    and r_hidden_out/s_hidden_out (down output) are shared; the 2048-wide side is per expert.
    Reading A14: down's input is per expert.  Reading A15: no router-weighted combine.
    ``col_blocks`` is None or a pair (blocks of the gate/up outputs, blocks of the down
    outputs).  Returns (gate [n, 2048], up [n, 2048], down [n, 6144]) float64.
    """
    cb_gu, cb_d = (None, None) if col_blocks is None else col_blocks
    g, u, d = [], [], []
    for k, e in enumerate(routed):
        ge, ue, de = layer.gate[e], layer.up[e], layer.down[e]
        g.append(forward(ge.code, ge.K, layer.r_hidden_in, ge.rout, layer.s_hidden_in, ge.s_out,
                         x_token, cb_gu, cb=getattr(ge, "cb", 1))[0])
        u.append(forward(ue.code, ue.K, layer.r_hidden_in, ue.rout, layer.s_hidden_in, ue.s_out,
                         x_token, cb_gu, cb=getattr(ue, "cb", 1))[0])
        d.append(forward(de.code, de.K, de.rin, layer.r_hidden_out, de.s_in, layer.s_hidden_out,
                         x_down[k:k + 1], cb_d, cb=getattr(de, "cb", 1))[0])
    return np.stack(g), np.stack(u), np.stack(d)


def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64.

    [EXLR8] calibration paragraph: the down projection's input is silu(gate x) times up x,
    elementwise.  For z below about -709 exp(-z) overflows to inf and the quotient is -0,
    the correctly rounded limit.
    """
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def moe_mlp_forward(layer, routed: Sequence[int], router_w: Sequence[float], x_token: np.ndarray,
                    return_act: bool = False):
    """Routed-expert MLP of one token, float64:  y = sum_k w_k * down_e(a_k),  e = routed[k],
    a_k = silu(gate_e(x)) * up_e(x)  (elementwise, [inter]).

    [EXLR8] calibration paragraph (a = silu(gate x) . up x, gate and up share the 6144-wide
    input x); width-manifest paragraph (gate/up stored per half: a half is 128 consecutive
    intermediate channels with its own width; down one width per expert); shared-rotation
    paragraph (the hidden side's vectors are one per layer).  Each linear is forward() above
    with that side's vectors: gate/up halves take the shared hidden input vectors and their
    own output vectors, down takes its own input vectors and the shared hidden output ones.
    gate_e(x) is the concatenation of its halves' outputs in half order.  Reading A21: the
    router weights are inputs (the pages fix no router), combined as a weighted sum of the
    experts' outputs.  Returns y [hidden] (and the activations a [n, inter] if asked).
    """
    x = np.atleast_2d(np.asarray(x_token))
    acts, y = [], np.zeros(layer.hidden)
    for k, e in enumerate(routed):
        cbk = lambda l: getattr(l, "cb", 1)  # each matrix's own codebook
        g = np.concatenate([forward(l.code, l.K, layer.r_hidden_in, l.rout, layer.s_hidden_in, l.s_out, x,
                                    cb=cbk(l))[0] for l in layer.gate[e]])
        u = np.concatenate([forward(l.code, l.K, layer.r_hidden_in, l.rout, layer.s_hidden_in, l.s_out, x,
                                    cb=cbk(l))[0] for l in layer.up[e]])
        a = silu(g) * u
        d = layer.down[e]
        y = y + float(router_w[k]) * forward(d.code, d.K, d.rin, layer.r_hidden_out, d.s_in,
                                             layer.s_hidden_out, a[None, :], cb=cbk(d))[0]
        acts.append(a)
    act = np.stack(acts) if acts else np.zeros((0, layer.inter))
    return (y, act) if return_act else y


# ----------------------------------------------------------------------------------------
# Test encoder: tail-biting Viterbi + packer (never on the product path)
# ----------------------------------------------------------------------------------------

def symbol_order(tiles: np.ndarray) -> np.ndarray:
    """[T, 16, 16] tile values -> [T, 256] in symbol order (x_s = T[r(s), c(s)])."""
    r, c = symbol_position(np.arange(256))
    return np.asarray(tiles)[:, r, c]


def viterbi_encode(targets: np.ndarray, K: int, batch: int = 16, cb: int = 1,
                   dtype=np.float64) -> np.ndarray:
    """Minimum squared-error tail-biting trellis paths: [T, 16, 16] -> states uint16 [T, 256].

    [EXLR8] tile-coding paragraph: a tile is a path through a 16-bit-state trellis, each
    weight contributing K new bits; the Viterbi search picks the path that minimises the
    tile's squared error against the MCG codebook.  The transition is
    n = ((p << K) | b) & 0xFFFF.  Reading A16 (the pages do not say how the circular
    constraint is searched): two passes.  Pass 1 runs with a free start and takes the
    best end state; its low 16-K bits O fix the wrap.  Pass 2 restricts the start to
    states whose high 16-K bits are O and the end to states whose low 16-K bits are O,
    which makes the path close on itself.  Ties go to the lowest index (argmin).

    cb = 2: the per-step values are the E4M3 codebook's ([EXLR8] E4M3 paragraph: the
    rounding happens inside the search).  ``dtype``: the arithmetic of the path costs.  Each
    step computes cost = best + (x - value)^2 as a subtraction, a multiplication and an
    addition, each rounded once in that type; with float32 the minima and argmins are the
    decisions a float32 search takes (reading A26).
    """
    x_all = symbol_order(targets).astype(dtype)
    table = codebook_table().astype(np.float64)
    if cb == 2:
        table = e4m3_round(table)
    cb = table.astype(dtype)
    lowbits = 16 - K
    mask_lo = (1 << lowbits) - 1
    n_all = np.arange(1 << 16)
    out = np.empty((x_all.shape[0], 256), np.uint16)

    def run(x, start_ok, end_ok):
        T = x.shape[0]
        d = x[:, 0, None] - cb[None, :]
        cost = d * d
        if start_ok is not None:
            cost = np.where(start_ok, cost, dtype(np.inf))
        back = np.empty((256, T, 1 << lowbits), np.uint8)
        for s in range(1, 256):
            c3 = cost.reshape(T, 1 << K, 1 << lowbits)  # [T, top K bits t, middle m]
            t_best = np.argmin(c3, axis=1)  # predecessor p = (t << lowbits) | m
            best = np.take_along_axis(c3, t_best[:, None, :], axis=1)[:, 0, :]
            back[s] = t_best
            d = x[:, s, None] - cb[None, :]
            cost = np.repeat(best, 1 << K, axis=1) + d * d
        if end_ok is not None:
            cost = np.where(end_ok, cost, dtype(np.inf))
        end = np.argmin(cost, axis=1)
        states = np.empty((T, 256), np.int64)
        states[:, 255] = end
        for s in range(255, 0, -1):
            m = states[:, s] >> K
            t = back[s][np.arange(T), m]
            states[:, s - 1] = (t.astype(np.int64) << lowbits) | m
        return states, end

    for a in range(0, x_all.shape[0], batch):
        x = x_all[a:a + batch]
        _, end1 = run(x, None, None)
        O = (end1 & mask_lo)[:, None]
        start_ok = (n_all[None, :] >> K) == O
        end_ok = (n_all[None, :] & mask_lo) == O
        st, _ = run(x, start_ok, end_ok)
        out[a:a + batch] = st.astype(np.uint16)
    return out


def pack_states(states: np.ndarray, K: int) -> np.ndarray:
    """Tail-biting state paths [T, 256] -> packed words int16 [T, 16K].

    Symbol s contributes its own K bits (the low K bits of its state) at stream bits
    sK .. sK+K-1, most significant first; the stream is cut into 32-bit words, most
    significant bit first, and each word is stored as two little-endian int16 halves
    (the inverse of ``stream_bits``).
    """
    st = np.asarray(states).astype(np.uint32)
    T = st.shape[0]
    sym = st & np.uint32((1 << K) - 1)  # [T, 256]
    shifts = np.arange(K - 1, -1, -1)
    bits = ((sym[:, :, None] >> shifts[None, None, :]) & 1).astype(np.uint8).reshape(T, 256 * K)
    be = np.packbits(bits, axis=-1)  # bytes, MSB first
    u = be.view(">u4").astype(np.uint32)  # [T, 8K]
    w = np.empty((T, 16 * K), np.uint16)
    w[:, 0::2] = (u & 0xFFFF).astype(np.uint16)
    w[:, 1::2] = (u >> 16).astype(np.uint16)
    return w.view(np.int16)


def rel_frobenius(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(a))


def rel_l2(y: np.ndarray, y_ref: np.ndarray) -> float:
    """Reading A17: ||y - y_ref||_2 / ||y_ref||_2 over the whole output tensor."""
    return rel_frobenius(y_ref, y)
