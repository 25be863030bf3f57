"""GPU parity of trellis_encode_tiles (the tail-biting Viterbi encoder) against the oracle.

The search's argmins are decisions, so the oracle runs its float32 search (the kernel's
precision and operations) and the paths must agree exactly: states, packed words, and
through trellis_decode_tiles the decoded weights.  A heavy-tailed, rotated matrix
encoded on the GPU must also land in the oracle's Shannon band."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from trellis_coded_bit_amd import binding as tb

from gpu_util import log_case, to_dev

pytestmark = pytest.mark.gpu


def _targets(seed, T):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, 16, 16)) * O.CODEBOOK_SCALE).astype(np.float32)


@pytest.mark.parametrize("cb", [1, 2])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_encode_matches_oracle_search(K, cb):
    log_case(f"encode K={K} cb={cb}")
    T = 10
    tgt = _targets(70 + 10 * K + cb, T)
    code, st = tb.trellis_encode_tiles(to_dev(tgt), K, cb, want_states=True)
    torch.cuda.synchronize()
    ref = O.viterbi_encode(tgt, K, cb=cb, dtype=np.float32)
    np.testing.assert_array_equal(st.cpu().numpy().view(np.uint16), ref)
    np.testing.assert_array_equal(code.cpu().numpy(), O.pack_states(ref, K))
    # the decoder reads back the path (tile words are independent of the tile's place)
    w, states = tb.trellis_decode_tiles(code.reshape(T, 1, 16 * K), K, want_states=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(states.cpu().numpy().view(np.uint16).reshape(T, 256), ref)


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


@pytest.mark.parametrize("K", [2, 3])
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
