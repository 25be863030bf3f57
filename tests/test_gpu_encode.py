"""GPU checks of trellis_encode_tiles (the tail-biting Viterbi encoder).

Primary, method-level ([EXLR8] tile-coding paragraph: each tile is a path through the
16-bit-state trellis that minimises the squared error against the codebook; any path of
least error is a correct result):
  * the GPU's states form a valid tail-biting path (consecutive states overlap in 16 - K
    bits, including the wrap from the last symbol to the first), its packed words are that
    path, and trellis_decode_tiles reads the same states back;
  * its float64 squared error is no larger than that of the oracle's float64 search
    (within 1e-5 relative);
  * a heavy-tailed rotated matrix encoded on the GPU lands in the Shannon band at K = 2, 3, 4.
Secondary: the paths equal the oracle's float32 search (same precision as the kernel; ties to
the lowest state index) bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb

from gpu_util import log_case, to_dev

pytestmark = pytest.mark.gpu


def _path_errors(states: np.ndarray, tiles: np.ndarray, cb: int) -> np.ndarray:
    """float64 squared error of each tile's path against its targets (symbol order)."""
    table = O.codebook_table().astype(np.float64)
    if cb == 2:
        table = O.e4m3_round(table)
    x = O.symbol_order(tiles).astype(np.float64)
    return ((x - table[states.astype(np.int64)]) ** 2).sum(axis=1)


def _assert_tail_biting(states: np.ndarray, K: int):
    st = states.astype(np.int64)
    low = (1 << (16 - K)) - 1
    nxt = np.roll(st, -1, axis=1)  # state s + 1, and state 0 after state 255
    assert np.array_equal(st & low, nxt >> K)


def _targets(seed, T):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, 16, 16)) * O.CODEBOOK_SCALE).astype(np.float32)


@pytest.mark.parametrize("cb", [1, 2])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_encode_paths_are_least_error_tail_biting_paths(K, cb):
    log_case(f"encode K={K} cb={cb}")
    T = 10
    tgt = _targets(70 + 10 * K + cb, T)
    code, st = tb.trellis_encode_tiles(to_dev(tgt), K, cb, want_states=True)
    torch.cuda.synchronize()
    st = st.cpu().numpy().view(np.uint16)
    _assert_tail_biting(st, K)
    np.testing.assert_array_equal(code.cpu().numpy(), O.pack_states(st, K))
    _, back = tb.trellis_decode_tiles(code.reshape(T, 1, 16 * K), K, want_states=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(back.cpu().numpy().view(np.uint16).reshape(T, 256), st)
    best = _path_errors(O.viterbi_encode(tgt, K, cb=cb, dtype=np.float64), tgt, cb)
    got = _path_errors(st, tgt, cb)
    assert np.all(got <= best * (1 + 1e-5)), (got / best).max()


@pytest.mark.parametrize("cb", [1, 2])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_encode_matches_float32_search(K, cb):
    """Secondary: the float32 search with the kernel's tie rule finds the same paths."""
    T = 10
    tgt = _targets(70 + 10 * K + cb, T)
    _, st = tb.trellis_encode_tiles(to_dev(tgt), K, cb, want_states=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.cpu().numpy().view(np.uint16), O.viterbi_encode(tgt, K, cb=cb, dtype=np.float32))


def test_encode_edge_targets():
    """Constant and all-zero tiles (massive ties: the lowest index must win everywhere)."""
    tgt = np.zeros((3, 16, 16), np.float32)
    tgt[1] = 1.84375  # the codebook value of the all-zero state
    tgt[2] = -3.0
    for K in (2, 4):
        code, st = tb.trellis_encode_tiles(to_dev(tgt), K, 1, want_states=True)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st.cpu().numpy().view(np.uint16), O.viterbi_encode(tgt, K, dtype=np.float32))
    assert tb.trellis_encode_tiles(torch.empty((0, 16, 16), device="cuda"), 2)[0].shape == (0, 32)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_encode_shannon_band(K):
    """[METAL] Shannon-bound paragraph / [EXLR8] rotation paragraphs: a Student-t matrix
    rotated with random signs and the Hadamard on both sides, scaled to the codebook's
    scale, encoded tile by tile on the GPU; the relative Frobenius error of the decode lies
    in (2^-K, 1.25 * 2^-K]."""
    rng = np.random.default_rng(99)
    W = rng.standard_t(3, size=(128, 128))
    d1, d2 = rng.choice([-1.0, 1.0], 128), rng.choice([-1.0, 1.0], 128)
    H = O.hadamard128()
    Wr = H @ (d1[:, None] * W * d2[None, :]) @ H
    Wr *= O.CODEBOOK_SCALE / Wr.std()
    tiles = Wr.reshape(8, 16, 8, 16).transpose(0, 2, 1, 3).reshape(64, 16, 16).astype(np.float32)
    code, _ = tb.trellis_encode_tiles(to_dev(tiles), K)
    w_hat, _ = tb.trellis_decode_tiles(code.reshape(8, 8, 16 * K), K)
    torch.cuda.synchronize()
    relf = O.rel_frobenius(Wr.astype(np.float32), w_hat.cpu().numpy().astype(np.float64))
    assert 2.0 ** -K < relf <= 1.25 * 2.0 ** -K, relf
