"""Pin of the oracle's fp32 -> bf16 rounding (oracle/params.py bf16_round).

bf16 keeps the top 16 bits of an IEEE binary32 value; rounding to nearest with
ties to even is the conversion PyTorch implements for torch.bfloat16, an
implementation independent of the oracle's integer formula.  The pin compares
bit patterns:

* on 10^6 random finite binary32 bit patterns (every exponent, subnormals
  included) and 10^6 normal values of the magnitudes the workloads use;
* on every exact tie (low 16 bits 0x8000) of every finite high half, where a
  ties-away or ties-to-odd mistake shows, and on the patterns one unit either
  side of each tie and at the ends of each rounding interval (0x0000, 0xFFFF);
* and states the tie rule itself: each exact tie lands on the even neighbour.
"""
import numpy as np
import torch

from oracle import params


def _torch_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return (t.view(torch.int16).numpy().astype(np.uint16).astype(np.uint32)) << 16


def _oracle_bits(x32):
    return params.bf16_round(np.ascontiguousarray(x32, np.float32)).view(np.uint32)


def _finite_highs():
    hi = np.arange(1 << 16, dtype=np.uint32)
    return hi[((hi >> 7) & 0xFF) != 0xFF]          # exponent field not all ones


def test_random_bit_patterns_match_library():
    rs = np.random.default_rng(11)
    bits = rs.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]      # finite values only
    x = bits.view(np.float32)
    assert np.array_equal(_oracle_bits(x), _torch_bits(x))


def test_workload_magnitudes_match_library():
    rs = np.random.default_rng(12)
    x = np.concatenate([rs.standard_normal(250_000) * s for s in (0.02, 1.0, 30.0, 1e-5)]).astype(np.float32)
    assert np.array_equal(_oracle_bits(x), _torch_bits(x))


def test_every_tie_and_its_neighbours_match_library():
    hi = _finite_highs()
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF):
        bits = (hi << 16) | np.uint32(low)
        x = bits.view(np.float32)
        assert np.array_equal(_oracle_bits(x), _torch_bits(x)), hex(low)


def test_ties_go_to_even():
    hi = _finite_highs()
    x = ((hi << 16) | np.uint32(0x8000)).view(np.float32)
    out = _oracle_bits(x) >> 16
    # the result is one of the two neighbours (hi or hi + 1) and the one with an even last bit
    assert np.all((out == hi) | (out == hi + 1))
    assert np.all((out & 1) == 0)
    # just below a tie rounds down, just above rounds up (magnitude-wise)
    below = _oracle_bits(((hi << 16) | np.uint32(0x7FFF)).view(np.float32)) >> 16
    above = _oracle_bits(((hi << 16) | np.uint32(0x8001)).view(np.float32)) >> 16
    assert np.array_equal(below, hi) and np.array_equal(above, hi + 1)
