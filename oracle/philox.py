"""Philox4x64-10 counter-based generator, written from its published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11, section 3 (the Philox family) with the
4x64 multipliers and Weyl key increments given there, 10 rounds.

TEST INFRASTRUCTURE: part of the oracle. Only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg may import it.

One Philox4x64 round maps a counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

where hi/lo are the upper/lower 64 bits of the 128-bit product. Between
rounds the key is bumped by the Weyl constants (W0, W1). Pure Python integers
make every step visible; no vectorisation, no shortcuts.

Uniform convention of this verifier (the pages leave the consumption order of
random numbers free: "Drafters and Speculative Decoding", section
"Distribution, seeded output and quality"): for request b and slot j
(j < gamma: acceptance test of proposal j; j == gamma: the single final draw),
    r = Philox4x64-10(counter = (j, b, offset, 0), key = (seed, 0)) word 0
    u = ((r >> 11) + 1) * 2**-53,   so u lies in (0, 1] with 53-bit resolution.
"""

MASK64 = (1 << 64) - 1

PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one counter block."""
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        hi0, lo0 = prod0 >> 64, prod0 & MASK64
        hi1, lo1 = prod1 >> 64, prod1 & MASK64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return (c0, c1, c2, c3)


def word_to_uniform(r):
    """Map a 64-bit word to u in (0, 1]: top 53 bits plus one, times 2^-53."""
    return ((int(r) >> 11) + 1) * 2.0 ** -53


def uniform(seed, offset, b, j):
    """The uniform for request b, slot j (see module docstring)."""
    return word_to_uniform(philox4x64_10((j, b, offset, 0), (seed, 0))[0])


def uniforms(seed, offset, B, gamma):
    """All B x (gamma+1) uniforms of one verifier call, as nested lists."""
    return [[uniform(seed, offset, b, j) for j in range(gamma + 1)] for b in range(B)]
