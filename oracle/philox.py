"""Philox4x64-10 and the ISD uniforms drawn from it.  Test infrastructure.

The pages say only that acceptance is a probabilistic min(1, p/q) test
("Introspective Diffusion Language Models", section "Inference & ISD"); they
name no generator.  The step uses the counter-based Philox4x64 generator
with 10 rounds, written here from its published definition (Salmon, Moraes,
Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):

* state: a 4-word counter and a 2-word key, 64-bit words;
* one round multiplies counter words 0 and 2 by two fixed odd constants,
  keeps the 128-bit products' high and low halves, and forms the new counter
  from the high halves xor-ed with the other two words and the key, and the
  low halves;
* between rounds the key is advanced by two Weyl constants (the golden ratio
  and sqrt(3)-1 in 64-bit fixed point).

ISD contract (the same on the GPU side, implemented there independently):

* key     = (seed mod 2**64, b)        b = sequence index in the batch
* counter = (i, 0, 0, 0)               i = draft position 0..K
* word 0 gives the ratio-test uniform u_i, word 1 the sampling uniform u'_i;
* a word w maps to the uniform (w >> 40) * 2**-24, a multiple of 2**-24 in
  [0, 1) that is exact in float32 and float64.

Pinned in tests/test_oracle_philox.py against numpy's own Philox bit
generator (also Philox4x64-10), after probing its counter convention.
"""

MASK64 = (1 << 64) - 1

# Round multipliers and key increments of Philox4x64 (SC'11, Table/Section on
# the Philox family).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def _mulhilo(a, b):
    prod = a * b
    return prod >> 64, prod & MASK64


def philox4x64_10(counter, key):
    """Return the 4 output words of Philox4x64 with 10 rounds."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def word_to_uniform(w):
    """Top 24 bits of a 64-bit word as a float in [0, 1)."""
    return float(int(w) >> 40) * (2.0 ** -24)


def isd_uniforms(seed, b, i):
    """(u_i, u'_i) for sequence ``b`` and draft position ``i`` under ``seed``."""
    w = philox4x64_10((i, 0, 0, 0), (seed, b))
    return word_to_uniform(w[0]), word_to_uniform(w[1])


def propose_uniform(seed, b, i):
    """Uniform for proposing draft ``i`` of sequence ``b``'s next step: word 0
    of the block at counter (i, 1, 0, 0) under key (seed, b), a stream apart
    from the acceptance uniforms (counter word 1 is 0 there)."""
    w = philox4x64_10((i, 1, 0, 0), (seed, b))
    return word_to_uniform(w[0])
