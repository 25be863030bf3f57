"""Pins for the CPU oracle against what the pages and mathematics fix (no GPU needed).

Each test names the fact it checks and where the fact comes from.  The oracle is never
checked against itself: each pin uses a second route (a hand derivation, the public PTX
fragment layout, scipy, Python's own binary16 packing, the rate-distortion bound, or an
encoder round trip).
"""
import math
import os
import struct

import numpy as np
import pytest
import scipy.linalg

import oracle as O
from trellis_coded_bit_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_code(rng, n_tiles, K):
    return rng.integers(0, 1 << 16, size=(n_tiles, 16 * K), dtype=np.uint16).view(np.int16)


# ---------------------------------------------------------------------------------------
# Codebook
# ---------------------------------------------------------------------------------------

def test_codebook_hand_derived_values():
    """tests/golden/codebook_hand.txt: values derived by hand from the printed constants."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "codebook_hand.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for st, hx, val in rows:
        s = int(st, 16)
        assert int(O.mcg_hash(np.array([s]))[0]) == int(hx, 16)
        assert float(O.codebook(np.array([s]))[0]) == float(val)


def _half_bits_to_float(h: int) -> float:
    return struct.unpack("<e", struct.pack("<H", h))[0]


def test_codebook_rounding_matches_python_binary16_packing():
    """The fp16 codebook value is one round-to-nearest-even of the exact half sum.

    Second route: Python's struct 'e' packing (IEEE-754 binary16, round-half-even), with the
    hash computed by Python integers.  Covers all 65536 states.
    """
    table = O.codebook_table()
    mult, mask, xor = 0xCBAC1FED, 0x8FFF8FFF, 0x3B603B60
    n_rounded = 0
    for s in range(1 << 16):
        v = ((s * mult) & 0xFFFFFFFF) & mask ^ xor
        exact = _half_bits_to_float(v & 0xFFFF) + _half_bits_to_float(v >> 16)
        ref = struct.unpack("<e", struct.pack("<e", exact))[0]
        got = float(table[s])
        assert got == ref, (hex(s), got, ref)
        n_rounded += ref != exact
    # the rounding is not vacuous: many states need it
    assert n_rounded > 10000


def test_codebook_statistics_match_codebook_scale():
    """[ESCHA] "How each claim was verified" item 3: EXL3's codebook_scale = 1.24371088.

    The std over all 65536 states must sit near it; each half is +-[2^-3, 2) by the forced
    exponent bits, so |value| < 4 and no value is subnormal except exact zeros.
    """
    t = O.codebook_table().astype(np.float64)
    assert abs(t.std() - O.CODEBOOK_SCALE) / O.CODEBOOK_SCALE < 0.005
    assert abs(t.mean()) < 0.01
    assert np.abs(t).max() < 4.0
    nz = np.abs(t[t != 0])
    assert nz.min() >= 2.0 ** -14  # no fp16 subnormals
    # masked halves always have exponent field 0b011xx (|half| in [1/8, 2))
    v = O.mcg_hash(np.arange(1 << 16))
    for half in (v & 0xFFFF, v >> 16):
        exp = (half >> 10) & 0x1F
        assert np.all((exp >= 12) & (exp <= 15))


# ---------------------------------------------------------------------------------------
# Bit layout
# ---------------------------------------------------------------------------------------

def test_states_hand_derived_tiles():
    """tests/golden/states_hand.txt: tiles with one non-zero symbol, their states derived by
    hand from the bit-layout definition (word pairing, most-significant-bit-first stream,
    window ending at the symbol's own K bits, circular) at K = 2, 3, 4."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "states_hand.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for K_s, words_s, states_s in rows:
        K = int(K_s)
        w = np.zeros((1, 16 * K), np.uint16)
        for item in words_s.split(","):
            i, v = item.split("=")
            w[0, int(i)] = int(v, 16)
        expect = np.zeros(256, np.int64)
        for item in states_s.split(","):
            i, v = item.split("=")
            expect[int(i)] = int(v, 16)
        got = O.tile_states(w.view(np.int16), K)[0].astype(np.int64)
        np.testing.assert_array_equal(got, expect, err_msg=f"K={K}")


def test_states_catch_swapped_word_halves():
    """The hand-derived case discriminates the pairing order: putting the set half in the
    other half of its 32-bit word (big-endian pairing) moves the symbol and changes the
    states (shown by decoding the swapped tile with the oracle)."""
    w = np.zeros((1, 32), np.uint16)
    w[0, 2] = 0x2000  # the golden K = 2 case's half in the wrong position
    st = O.tile_states(w.view(np.int16), 2)[0]
    assert st[17] == 0 and st[24] == 0 and np.count_nonzero(st) > 0


def test_states_special_streams():
    """Closed forms: an all-zero stream gives state 0 everywhere, all-ones gives 0xFFFF.

    A single set stream bit p appears in exactly the 16 windows that cover it, at the
    position that puts later stream bits lower (MSB-first).
    """
    for K in (2, 3, 4):
        z = np.zeros((1, 16 * K), np.int16)
        assert np.all(O.tile_states(z, K) == 0)
        o = np.full((1, 16 * K), -1, np.int16)
        assert np.all(O.tile_states(o, K) == 0xFFFF)
        # set the most significant bit of u32[0] = stream bit 0 = bit 15 of word 1
        w = np.zeros((1, 16 * K), np.uint16)
        w[0, 1] = 0x8000
        st = O.tile_states(w.view(np.int16), K)[0].astype(np.int64)
        nz = np.nonzero(st)[0]
        # stream bit 0 belongs to symbol 0; it is the top (first) bit of symbol 0's own K bits
        assert st[0] == 1 << (K - 1)
        # it stays in the window for the next floor((16-K)/K) symbols, moving up K bits a step
        for d in range(1, 20):
            pos = (K - 1) + d * K
            expect = (1 << pos) if pos < 16 else 0
            assert st[d] == expect, (K, d, st[d], expect)
        assert set(nz.tolist()) <= set(range(0, 16))


@pytest.mark.parametrize("K", [2, 3, 4])
def test_overlap_invariant_including_wrap(K):
    """[ESCHA] "How each claim was verified" item 1: the low 16-K bits of state t equal the
    high 16-K bits of state t+1 -- here for every pair including the wrap 255 -> 0."""
    rng = np.random.default_rng(100 + K)
    st = O.tile_states(_rand_code(rng, 64, K), K).astype(np.int64)
    lo = st & ((1 << (16 - K)) - 1)
    hi = np.roll(st, -1, axis=1) >> K
    assert np.array_equal(lo, hi)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_constant_window_offset_is_caught(K):
    """The overlap test is blind to a constant window offset ([ESCHA] item 1 caveat), so the
    planted offset must be caught by a different pin: the K=2 lane rule, or the round trip
    with the encoder below.  Here: an off-by-one-symbol decode still satisfies the overlap
    invariant but disagrees with the true states."""
    rng = np.random.default_rng(7)
    st = O.tile_states(_rand_code(rng, 8, K), K).astype(np.int64)
    shifted = np.roll(st, 1, axis=1)  # planted mistake: constant one-symbol offset
    lo = shifted & ((1 << (16 - K)) - 1)
    assert np.array_equal(lo, np.roll(shifted, -1, axis=1) >> K)  # invariant still holds
    assert not np.array_equal(shifted, st)


# ---------------------------------------------------------------------------------------
# Permutation
# ---------------------------------------------------------------------------------------

def test_permutation_is_bijection_and_matches_closed_form():
    """[METAL] tile paragraph closed form: t = 4(4(c&7)+q) + 2((c>>3)&1) + rh,
    r = 8rh + 2q + e, with s = 2t + e (reading A6)."""
    r, c = O.symbol_position(np.arange(256))
    assert len(set(zip(r.tolist(), c.tolist()))) == 256
    for s in range(256):
        rr, cc = int(r[s]), int(c[s])
        e = rr & 1
        rh = rr >> 3
        q = (rr & 7) >> 1
        t = 4 * (4 * (cc & 7) + q) + 2 * ((cc >> 3) & 1) + rh
        assert 2 * t + e == s


def test_permutation_matches_public_mma_b_fragment():
    """The stored order is the B-operand fragment of the public PTX mma.m16n8k16 layout:
    in a warp, thread T (group g = T>>2, thread-in-group i = T&3) holds, for each of the two
    n8 halves h, the elements (k = 2i, 2i+1, 2i+8, 2i+9; n = 8h + g).  [ESCHA] "Bit layout":
    lane L covers symbols 8L..8L+7.  So lane L's symbol 8L + 4h + 2*rh + e sits at
    row 2i + e + 8rh, column 8h + g."""
    r, c = O.symbol_position(np.arange(256))
    for L in range(32):
        g, i = L >> 2, L & 3
        for h in range(2):
            for rh in range(2):
                for e in range(2):
                    s = 8 * L + 4 * h + 2 * rh + e
                    assert (int(r[s]), int(c[s])) == (2 * i + e + 8 * rh, 8 * h + g)


def test_tile_placement():
    """[ESCHA] "Bit layout": code[i, j] maps to W_inner[16i:16i+16, 16j:16j+16], i major."""
    rng = np.random.default_rng(3)
    code = _rand_code(rng, 3 * 5, 2).reshape(3, 5, 32)
    w = O.decode_tiles(code, 2)
    assert w.shape == (48, 80) and w.dtype == np.float16
    r, c = O.symbol_position(np.arange(256))
    for i in range(3):
        for j in range(5):
            vals = O.codebook(O.tile_states(code[i, j], 2))
            blk = w[16 * i:16 * i + 16, 16 * j:16 * j + 16]
            for s in range(0, 256, 17):
                assert blk[r[s], c[s]] == vals[s]


# ---------------------------------------------------------------------------------------
# Hadamard and the forward
# ---------------------------------------------------------------------------------------

def test_hadamard_properties_and_library_match():
    """[ESCHA] "Reconstruction": normalised Sylvester H_128, symmetric, orthogonal, its own
    inverse.  Second route: scipy.linalg.hadamard (Sylvester construction)."""
    H = O.hadamard128()
    np.testing.assert_array_equal(H, H.T)
    np.testing.assert_allclose(H @ H, np.eye(128), atol=1e-13)
    np.testing.assert_allclose(np.abs(H), 2.0 ** -3.5, rtol=1e-15)
    np.testing.assert_allclose(H, scipy.linalg.hadamard(128) / math.sqrt(128), rtol=0, atol=0)
    z = np.random.default_rng(0).standard_normal((3, 384))
    np.testing.assert_allclose(O.had_blocks(O.had_blocks(z)), z, atol=1e-12)


def test_forward_equals_dense_reconstruction_single_k2():
    """The activation-side factoring ([METAL] reconstruction paragraph) must equal x @ W with
    the dense W of [ESCHA] "Reconstruction" (signs/scales folded).  Dense side built with
    scipy's Hadamard, independently of the oracle's rotation code."""
    wl = synth.single_k2(0)
    lin, x = wl.layers["w"], wl.xs["w"]
    y = O.forward_linear(lin, x)
    w_hat = O.decode_tiles(lin.code, lin.K).astype(np.float64)
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    hl = np.kron(np.eye(512 // 128), H)
    hr = np.kron(np.eye(256 // 128), H)
    su = lin.rin.astype(np.float64) * lin.s_in
    sv = lin.rout.astype(np.float64) * lin.s_out
    W = su[:, None] * (hl @ w_hat @ hr) * sv[None, :]
    ref = x.astype(np.float64) @ W
    assert O.rel_l2(y, ref) < 1e-13
    # and the oracle's own dense form agrees
    assert O.rel_l2(x.astype(np.float64) @ O.dense_weight(lin.code, 2, lin.rin, lin.rout, lin.s_in, lin.s_out), ref) < 1e-13


def test_forward_column_blocks_and_orthogonality():
    """forward() restricted to column blocks equals the full forward on those columns, and
    ||y / sv|| = ||x_h @ W_hat|| because H is orthogonal."""
    rng = np.random.default_rng(5)
    lin = synth.make_linear(np.random.SeedSequence(9), 3, 256, 384)
    x = rng.standard_normal((2, 256)).astype(np.float16)
    y = O.forward_linear(lin, x)
    yc = O.forward_linear(lin, x, col_blocks=[2, 0])
    np.testing.assert_allclose(yc, np.concatenate([y[:, 256:384], y[:, 0:128]], axis=1), rtol=1e-12)
    su = lin.rin.astype(np.float64) * lin.s_in
    sv = lin.rout.astype(np.float64) * lin.s_out
    xh = O.had_blocks(x.astype(np.float64) * su)
    y_pre = xh @ O.decode_tiles(lin.code, 3).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(y / sv, axis=1), np.linalg.norm(y_pre, axis=1), rtol=1e-12)


# ---------------------------------------------------------------------------------------
# Encoder round trip and the Shannon band
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("K", [2, 3, 4])
def test_viterbi_pack_decode_round_trip(K):
    """decode(pack(path)) == codebook(path) exactly, and the packed path is a valid
    tail-biting path (the decoded states are the encoder's states)."""
    rng = np.random.default_rng(20 + K)
    tgt = rng.standard_normal((6, 16, 16)) * O.CODEBOOK_SCALE
    path = O.viterbi_encode(tgt, K)
    words = O.pack_states(path, K)
    st = O.tile_states(words, K)
    np.testing.assert_array_equal(st, path)
    # placed into the tile, the decoded values are the codebook values at the path
    dec = O.decode_tiles(words.reshape(6, 1, 16 * K), K)
    assert dec.shape == (96, 16)
    r, c = O.symbol_position(np.arange(256))
    for t in range(6):
        np.testing.assert_array_equal(dec[16 * t + r, c], O.codebook(path[t]))


@pytest.mark.parametrize("K", [2, 4])
def test_viterbi_e4m3_codebook_and_float32_search(K):
    """cb = 2: the path's decoded values (E4M3 decode) are the E4M3 codebook values at the
    path, and no path scores better under that codebook than the search's (checked against
    the cb = 1 path re-scored with E4M3 values).  float32 search: a valid tail-biting path
    whose float64 cost is within 1e-5 of the float64 search's."""
    rng = np.random.default_rng(40 + K)
    tgt = (rng.standard_normal((5, 16, 16)) * O.CODEBOOK_SCALE).astype(np.float32)
    x = O.symbol_order(tgt).astype(np.float64)
    v16 = O.codebook_table().astype(np.float64)
    v8 = O.e4m3_round(v16)
    p8 = O.viterbi_encode(tgt, K, cb=2, dtype=np.float32)
    words = O.pack_states(p8, K)
    np.testing.assert_array_equal(O.tile_states(words, K), p8)
    dec = O.decode_tiles(words.reshape(5, 1, 16 * K), K, cb=2).astype(np.float64)
    r, c = O.symbol_position(np.arange(256))
    for t in range(5):
        np.testing.assert_array_equal(dec[16 * t + r, c], v8[p8[t]])
    p16 = O.viterbi_encode(tgt, K)
    cost8 = ((x - v8[p8]) ** 2).sum(1)
    assert np.all(cost8 <= ((x - v8[p16]) ** 2).sum(1) * (1 + 1e-6))
    p32 = O.viterbi_encode(tgt, K, dtype=np.float32)
    np.testing.assert_array_equal(O.tile_states(O.pack_states(p32, K), K), p32)
    c32, c64 = ((x - v16[p32]) ** 2).sum(1), ((x - v16[p16]) ** 2).sum(1)
    np.testing.assert_allclose(c32, c64, rtol=1e-5)


def _shannon_relf(K, n_tiles=32, planted_offset=False):
    """[METAL] Shannon-bound paragraph, [EXLR8] rotation paragraphs: rotate a heavy-tailed
    matrix with random signs and the Hadamard on both sides, scale it to the codebook's
    scale, encode every tile, decode, and measure the relative Frobenius error."""
    rng = np.random.default_rng(1234)
    W = rng.standard_t(3, size=(128, 128))
    d1 = rng.choice([-1.0, 1.0], size=128)
    d2 = rng.choice([-1.0, 1.0], size=128)
    H = O.hadamard128()
    Wr = H @ (d1[:, None] * W * d2[None, :]) @ H
    Wr *= O.CODEBOOK_SCALE / Wr.std()
    tiles = Wr.reshape(8, 16, 8, 16).transpose(0, 2, 1, 3).reshape(64, 16, 16)[:n_tiles]
    words = O.pack_states(O.viterbi_encode(tiles, K), K)
    states = O.tile_states(words, K)
    if planted_offset:
        states = np.roll(states, 1, axis=1)
    dec = O.codebook(states).astype(np.float64)
    return O.rel_frobenius(O.symbol_order(tiles), dec)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_shannon_band(K):
    """Rate-distortion bound for a Gaussian source at R = K bits: relF >= 2^-K; a trellis
    code lands a few percent above it.  Accepted band: 2^-K < relF <= 1.25 * 2^-K."""
    relf = _shannon_relf(K)
    assert 2.0 ** -K < relf <= 1.25 * 2.0 ** -K, relf


def test_shannon_band_catches_offset_decode():
    """A decode with a constant one-symbol window offset leaves the band by far."""
    assert _shannon_relf(2, n_tiles=8, planted_offset=True) > 1.0


# ---------------------------------------------------------------------------------------
# E4M3 codebook and FP8 prefill ([EXLR8] E4M3 paragraph)
# ---------------------------------------------------------------------------------------

def test_e4m3_hand_derived_values():
    """From the OCP E4M3 definition (bias 7, 3 mantissa bits, subnormal step 2^-9, max 448):
    ties go to the even code, values past 448 saturate, a negative value keeps its sign."""
    cases = [
        (1.0625, 1.0),          # halfway 1.0 (code 0x38, even) / 1.125 (0x39)
        (1.1875, 1.25),         # halfway 1.125 (0x39) / 1.25 (0x3A, even)
        (2.0 ** -10, 0.0),      # halfway 0 (even) / 2^-9 (code 1)
        (3 * 2.0 ** -10, 2.0 ** -8),  # halfway 2^-9 (code 1) / 2^-8 (code 2, even)
        (2.0 ** -6, 2.0 ** -6), # smallest normal, exact
        (0.3, 0.3125),          # [0.25, 0.5) has step 1/32: 0.28125 / 0.3125, nearer the latter
        (448.0, 448.0), (464.0, 448.0), (500.0, 448.0), (1e9, 448.0), (-500.0, -448.0),
        (1.84375, 1.875),       # codebook value of the all-zero state
        (0.85009765625, 0.875), # codebook value of state 0xFFFF
    ]
    for v, want in cases:
        assert O.e4m3_round(v) == want, v
    assert np.signbit(O.e4m3_round(-2.0 ** -11)) and O.e4m3_round(-2.0 ** -11) == 0.0
    assert O.e4m3_codes(448.0) == 0x7E and O.e4m3_codes(-1.0) == 0xB8
    m = O.e4m3_magnitudes()
    assert len(m) == 127 and np.all(np.diff(m) > 0) and m[1] == 2.0 ** -9


def test_e4m3_matches_library_cast_on_every_fp16():
    """torch's float8_e4m3fn cast (round to nearest even) agrees on every finite fp16 value
    of magnitude <= 448; above it torch does not saturate, so that range is checked by the
    definition: everything from 448 up maps to 448."""
    import torch
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float64)
    fin = h[np.isfinite(h)]
    inr = fin[np.abs(fin) <= 448]
    ref = torch.from_numpy(inr).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_codes(inr), ref)
    big = fin[np.abs(fin) > 448]
    np.testing.assert_array_equal(O.e4m3_round(big), np.sign(big) * 448.0)


def test_codebook_e4m3_table():
    st = np.arange(1 << 16, dtype=np.uint32)
    v16 = O.codebook(st).astype(np.float64)
    v8 = O.e4m3_value(O.codebook_e4m3(st))
    # every value is the E4M3 value nearest the fp16 one: within half a step of it
    step = np.where(np.abs(v8) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v8), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(v8 - v16) <= step / 2 + 1e-15)
    assert np.all(np.abs(v8) <= 4) and np.max(np.abs(v8)) == 4.0  # |fp16 value| <= 3.9502 rounds up to 4
    assert O.e4m3_value(O.codebook_e4m3(np.array([0], np.uint32)))[0] == 1.875
    # decode of the cb=2 variant is the E4M3 rounding of the cb=1 decode, tile by tile
    code = synth.make_linear(np.random.SeedSequence(31), 3, 64, 48).code
    np.testing.assert_array_equal(O.decode_tiles(code, 3, cb=2).astype(np.float64),
                                  O.e4m3_round(O.decode_tiles(code, 3).astype(np.float64)))
    np.testing.assert_array_equal(O.e4m3_value(O.decode_tiles_e4m3(code, 3)),
                                  O.decode_tiles(code, 3, cb=2).astype(np.float64))


def test_fp8_prefill_one_hot_rotation():
    """x chosen so that had(x*su) is the k-th unit vector: its row scale is 1/448, its code
    is exactly 448 at k, and y must be had(row k of the E4M3 weights) * sv."""
    lin = synth.make_linear(np.random.SeedSequence(32), 2, 256, 256)
    lin.cb = 2
    su = lin.rin.astype(np.float64) * lin.s_in
    sv = lin.rout.astype(np.float64) * lin.s_out
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    for k in (0, 77, 200):
        e = np.zeros(256)
        e[k] = 1.0
        x = (np.kron(np.eye(2), H) @ e) / su
        y = O.forward_linear(lin, x[None, :], act_e4m3=True)[0]
        w8 = O.decode_tiles(lin.code, 2, cb=2).astype(np.float64)
        ref = (np.kron(np.eye(2), H) @ w8[k]) * sv
        assert O.rel_l2(y, ref) < 1e-12, k
    # two-hot: xh = e_3 + 0.6 e_150.  Row scale 1/448; 0.6 * 448 = 268.8 lies between the
    # E4M3 values 256 and 288 (step 32 in [256, 448]) and rounds to 256, so y_pre =
    # w8[3] + (256/448) w8[150].
    e = np.zeros(256)
    e[3], e[150] = 1.0, 0.6
    x = (np.kron(np.eye(2), H) @ e) / su
    y = O.forward_linear(lin, x[None, :], act_e4m3=True)[0]
    ref = (np.kron(np.eye(2), H) @ (w8[3] + (256.0 / 448.0) * w8[150])) * sv
    assert O.rel_l2(y, ref) < 1e-12


def test_fp8_prefill_scaling_and_quantisation_band():
    """Powers of two pass through the row scale exactly; a zero row gives zero; against the
    unquantised cb=2 forward the activation rounding costs 1-5 % relative L2 (E4M3 keeps 3
    mantissa bits: relative rounding error up to 2^-4 per element)."""
    lin = synth.make_linear(np.random.SeedSequence(33), 3, 384, 256)
    lin.cb = 2
    x = synth.make_x(np.random.SeedSequence(34), 3, 384).astype(np.float64)
    x[1] = 0.0
    y = O.forward_linear(lin, x, act_e4m3=True)
    np.testing.assert_allclose(O.forward_linear(lin, 8.0 * x, act_e4m3=True), 8.0 * y, rtol=1e-13, atol=0)
    assert np.all(y[1] == 0)
    exact = O.forward_linear(lin, x)
    for r in (0, 2):
        assert 0.005 < O.rel_l2(y[r], exact[r]) < 0.05


# ---------------------------------------------------------------------------------------
# Routed-expert MLP ([EXLR8] calibration and width-manifest paragraphs)
# ---------------------------------------------------------------------------------------

def _small_mlp(seed=0, halves=2):
    return synth.moe_mlp_layer(seed, n_experts=4, hidden=256, inter=256, halves=halves)


def test_silu_closed_forms_and_library():
    """silu(z) = z * sigmoid(z): exact points, the odd-part identity silu(z) - silu(-z) = z,
    the overflow limits, and scipy's logistic function."""
    import scipy.special
    assert O.silu(0.0) == 0.0
    assert O.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)  # sigmoid(ln 3) = 3/4
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z) - O.silu(-z), z, atol=1e-13)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    big = O.silu(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 800.0 and np.all(np.isfinite(big))


def _dense(lin, rin, s_in, rout, s_out):
    """Dense W [in, out] from the decoded tiles, built with scipy's Hadamard."""
    H = scipy.linalg.hadamard(128) / math.sqrt(128)
    w_hat = O.decode_tiles(lin.code, lin.K).astype(np.float64)
    hl = np.kron(np.eye(w_hat.shape[0] // 128), H)
    hr = np.kron(np.eye(w_hat.shape[1] // 128), H)
    su = rin.astype(np.float64) * s_in
    sv = rout.astype(np.float64) * s_out
    return su[:, None] * (hl @ w_hat @ hr) * sv[None, :]


def test_moe_mlp_equals_dense_composition():
    """The routed MLP equals sum_k w_k (silu(x Wg) * (x Wu)) Wd with dense matrices built
    independently: gate/up from their halves side by side with the shared hidden input
    vectors, down with the shared hidden output vectors."""
    import scipy.special
    L = _small_mlp(0)
    routed, w = [2, 0, 3], [0.5, 0.3, 0.2]
    x = synth.make_x(np.random.SeedSequence(11), 1, 256)
    y, act = O.moe_mlp_forward(L, routed, w, x, return_act=True)
    xf = x.astype(np.float64)
    ref = np.zeros((1, 256))
    for k, e in enumerate(routed):
        Wg = np.hstack([_dense(l, L.r_hidden_in, L.s_hidden_in, l.rout, l.s_out) for l in L.gate[e]])
        Wu = np.hstack([_dense(l, L.r_hidden_in, L.s_hidden_in, l.rout, l.s_out) for l in L.up[e]])
        d = L.down[e]
        Wd = _dense(d, d.rin, d.s_in, L.r_hidden_out, L.s_hidden_out)
        g, u = xf @ Wg, xf @ Wu
        a = g * scipy.special.expit(g) * u
        assert O.rel_l2(act[k], a[0]) < 1e-12
        ref += w[k] * (a @ Wd)
    assert O.rel_l2(y, ref[0]) < 1e-12


def _small_moe(seed=0):
    """A 4-expert MoE layer at hidden 256 / inner 128 whose per-expert hidden-side vectors
    (which moe_forward must NOT use) differ from the shared ones."""
    return synth.moe_layer(seed, n_experts=4, hidden=256, inner=128)


def test_moe_forward_equals_dense_matrices():
    """[EXLR8] shared-rotation paragraph: every expert's hidden side uses the layer's one
    vector pair.  Per routed expert, gate/up outputs equal x Wg and x Wu and the down output
    x_k Wd, with dense matrices built independently (scipy's Hadamard, _dense) from each
    expert's code: gate/up with the SHARED hidden input vectors on the input side and the
    expert's own on the 128-wide output side; down with the expert's own input vectors and
    the SHARED hidden output vectors."""
    L = _small_moe(0)
    routed = [3, 1, 2]
    x = synth.make_x(np.random.SeedSequence(21), 1, 256)
    xd = synth.make_x(np.random.SeedSequence(22), 3, 128)
    g, u, d = O.moe_forward(L, routed, x, xd)
    xf, xdf = x.astype(np.float64), xd.astype(np.float64)
    for k, e in enumerate(routed):
        ge, ue, de = L.gate[e], L.up[e], L.down[e]
        Wg = _dense(ge, L.r_hidden_in, L.s_hidden_in, ge.rout, ge.s_out)
        Wu = _dense(ue, L.r_hidden_in, L.s_hidden_in, ue.rout, ue.s_out)
        Wd = _dense(de, de.rin, de.s_in, L.r_hidden_out, L.s_hidden_out)
        assert O.rel_l2(g[k], (xf @ Wg)[0]) < 1e-12
        assert O.rel_l2(u[k], (xf @ Wu)[0]) < 1e-12
        assert O.rel_l2(d[k], (xdf[k:k + 1] @ Wd)[0]) < 1e-12


def test_moe_forward_pin_catches_swapped_side_vectors():
    """The pin above discriminates: had moe_forward used the experts' own hidden-side vectors
    instead of the shared ones (or swapped which side is shared), its outputs would differ
    from the dense reference by far more than rounding."""
    L = _small_moe(1)
    e = 2
    x = synth.make_x(np.random.SeedSequence(23), 1, 256)
    xd = synth.make_x(np.random.SeedSequence(24), 1, 128)
    g, _, d = O.moe_forward(L, [e], x, xd)
    ge, de = L.gate[e], L.down[e]
    wrong_in = _dense(ge, ge.rin, ge.s_in, ge.rout, ge.s_out)              # per-expert hidden input side
    wrong_side = _dense(ge, L.r_hidden_in, L.s_hidden_in, L.r_hidden_out[:128], L.s_hidden_out[:128])
    wrong_out = _dense(de, de.rin, de.s_in, de.rout, de.s_out)             # per-expert hidden output side
    xf = x.astype(np.float64)
    assert O.rel_l2(g[0], (xf @ wrong_in)[0]) > 0.05
    assert O.rel_l2(g[0], (xf @ wrong_side)[0]) > 0.05
    assert O.rel_l2(d[0], (xd.astype(np.float64) @ wrong_out)[0]) > 0.05


def test_forward_decoded_is_forward():
    """forward_decoded(decode_tiles(code)) is forward(code): the same definition evaluated
    in the same float64 order (a refactoring check)."""
    lin = synth.make_linear(np.random.SeedSequence(31), 3, 2048, 384)
    x = synth.make_x(np.random.SeedSequence(32), 3, 2048)
    a = O.forward_linear(lin, x)
    b = O.forward_decoded(O.decode_tiles(lin.code, 3), lin.rin, lin.rout, lin.s_in, lin.s_out, x)
    np.testing.assert_array_equal(a, b)


def test_moe_mlp_halves_are_consecutive_channel_slices():
    """Gate/up stored as two 128-channel halves (same width) give the same MLP as one
    full-width matrix whose column tiles and output vectors are those halves side by side."""
    import dataclasses
    L2 = _small_mlp(1, halves=2)
    gate, up = [], []
    for e in range(4):
        full = []
        for halves in (L2.gate[e], L2.up[e]):
            K = 3
            parts = [dataclasses.replace(h, K=K, code=synth.make_linear(np.random.SeedSequence([e, i, 7]), K, 256, 128).code)
                     for i, h in enumerate(halves)]
            full.append(parts)
        gate.append(full[0])
        up.append(full[1])
    Lh = dataclasses.replace(L2, gate=gate, up=up)

    def merged(halves):
        a, b = halves
        return dataclasses.replace(a, out_features=256, code=np.concatenate([a.code, b.code], axis=1),
                                   rout=np.concatenate([a.rout, b.rout]), s_out=np.concatenate([a.s_out, b.s_out]))
    L1 = dataclasses.replace(Lh, halves=1, gate=[[merged(g)] for g in gate], up=[[merged(u)] for u in up])
    x = synth.make_x(np.random.SeedSequence(12), 1, 256)
    y2, a2 = O.moe_mlp_forward(Lh, [1, 3], [0.6, 0.4], x, return_act=True)
    y1, a1 = O.moe_mlp_forward(L1, [1, 3], [0.6, 0.4], x, return_act=True)
    np.testing.assert_allclose(a2, a1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y2, y1, rtol=1e-12, atol=1e-12)
    # swapping the two halves of every expert changes the result
    Ls = dataclasses.replace(Lh, gate=[g[::-1] for g in gate], up=[u[::-1] for u in up])
    assert O.rel_l2(O.moe_mlp_forward(Ls, [1, 3], [0.6, 0.4], x), y1) > 0.1


def test_moe_mlp_linear_in_router_weights_and_order_free():
    L = _small_mlp(2)
    x = synth.make_x(np.random.SeedSequence(13), 1, 256)
    routed, w = [3, 1, 2], np.array([0.2, 0.7, 0.1])
    y = O.moe_mlp_forward(L, routed, w, x)
    parts = [O.moe_mlp_forward(L, [e], [1.0], x) for e in routed]
    np.testing.assert_allclose(y, sum(wk * p for wk, p in zip(w, parts)), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.moe_mlp_forward(L, routed[::-1], w[::-1], x), y, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O.moe_mlp_forward(L, routed, 2 * w, x), 2 * y, rtol=1e-12, atol=1e-12)
    y0, a0 = O.moe_mlp_forward(L, [], [], x, return_act=True)
    assert np.all(y0 == 0) and a0.shape == (0, 256)


# ---------------------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------------------

def test_synth_shapes_and_determinism():
    a = synth.single_k2(0)
    b = synth.single_k2(0)
    la, lb = a.layers["w"], b.layers["w"]
    assert la.code.shape == (32, 16, 32) and la.code.dtype == np.int16
    np.testing.assert_array_equal(la.code, lb.code)
    np.testing.assert_array_equal(a.xs["w"], b.xs["w"])
    assert np.all(la.s_in == 1.0) and np.all(la.s_out == 1.0)
    assert la.rin.dtype == np.float16 and 0.5 <= la.rin.min() and la.rin.max() <= 1.5
    assert la.code_bytes == 32768
    m = synth.moe_layer(0, experts=[3])
    assert m.gate[3].code.shape == (6144 // 16, 2048 // 16, 16 * int(m.K[3]))
    assert m.down[3].code.shape == (2048 // 16, 6144 // 16, 16 * int(m.K[3]))
    r = synth.moe_routes(0, 4)
    assert r.shape == (4, 8) and all(len(set(row)) == 8 for row in r.tolist())
    frac = np.bincount(synth.moe_layer(0, experts=[]).K, minlength=5)[2:] / 256
    assert np.all(np.abs(frac - np.array([0.3, 0.5, 0.2])) < 0.1)
