"""Pins for the oracle's Philox4x64-10 against numpy's Philox bit generator.

numpy's ``Philox`` is the same Philox4x64 with 10 rounds.  Its
``random_raw`` advances the 256-bit counter *before* producing a block, so the
block for counter c comes out of a generator seeded with counter c - 1.
"""

import numpy as np
import pytest

from oracle.philox import MASK64, isd_uniforms, philox4x64_10, word_to_uniform


def _numpy_block(counter, key):
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = [(c >> (64 * i)) & MASK64 for i in range(4)]
    bg = np.random.Philox(counter=np.array(words, dtype=np.uint64),
                          key=np.array([int(k) & MASK64 for k in key], dtype=np.uint64))
    return tuple(int(x) for x in bg.random_raw(4))


def test_numpy_counter_convention():
    # numpy increments first: seeding with counter 0 yields the block of counter 1.
    bg = np.random.Philox(counter=np.zeros(4, dtype=np.uint64), key=np.zeros(2, dtype=np.uint64))
    assert tuple(int(x) for x in bg.random_raw(4)) == philox4x64_10((1, 0, 0, 0), (0, 0))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((MASK64,) * 4, (MASK64, MASK64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
    ((7, 0, 0, 0), (12345, 3)),
    ((1, 2, 3, 4), (2 ** 63 + 5, 2 ** 40)),
])
def test_blocks_match_numpy(counter, key):
    assert philox4x64_10(counter, key) == _numpy_block(counter, key)


def test_random_blocks_match_numpy():
    rng = np.random.default_rng(3)
    for _ in range(200):
        counter = tuple(int(x) for x in rng.integers(0, 2 ** 63, 4)) if rng.random() < 0.5 else \
            (int(rng.integers(0, 64)), 0, 0, 0)
        key = (int(rng.integers(0, 2 ** 63)) * 2 + 1, int(rng.integers(0, 1 << 20)))
        assert philox4x64_10(counter, key) == _numpy_block(counter, key)


def test_uniform_mapping():
    assert word_to_uniform(0) == 0.0
    assert word_to_uniform(MASK64) == (2 ** 24 - 1) / 2 ** 24
    assert word_to_uniform(1 << 40) == 2.0 ** -24
    assert word_to_uniform((1 << 40) - 1) == 0.0
    rng = np.random.default_rng(4)
    for w in rng.integers(0, 2 ** 63, 1000):
        u = word_to_uniform(int(w) * 2)
        assert 0.0 <= u < 1.0 and (u * 2 ** 24).is_integer()
        assert np.float32(u) == u  # exact in float32


def test_isd_uniforms_use_words_0_and_1():
    seed, b, i = 0xDEADBEEF12345678, 5, 2
    w = _numpy_block((i, 0, 0, 0), (seed, b))
    assert isd_uniforms(seed, b, i) == (word_to_uniform(w[0]), word_to_uniform(w[1]))


def test_uniforms_are_uniform():
    # 24-bit uniforms from consecutive counters/keys look uniform (KS test).
    from scipy import stats
    us = [isd_uniforms(11, b, i)[k] for b in range(500) for i in range(4) for k in range(2)]
    assert stats.kstest(us, "uniform").pvalue > 1e-3
