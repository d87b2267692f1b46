"""Philox4x64-10, written from its published definition.

Source: J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers: As
Easy as 1, 2, 3", SC'11, section 3.2 (the Philox S-box and key schedule) and
table 2 (round counts and constants for Philox-4x64).

One round maps a counter (c0, c1, c2, c3) under key (k0, k1) to
    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
with 128-bit products split into hi/lo 64-bit halves.  Between rounds the key
is bumped by the Weyl constants (W0, W1) modulo 2^64.  Ten rounds.

How the verify path uses it (the configs ask for "a seeded Philox stream" and
the pages leave the rest open; this is the reading taken):
    key     = (seed, 0)
    counter = (slot, sequence b, round, tag 0)
    u       = (word0 >> 40) * 2^-24, a 24-bit uniform in [0, 1), exact in fp32.
Chain: slot j < gamma is the accept uniform of draft j+1; slot gamma draws the
resampled or bonus token.  Tree with T nodes: node c >= 1 uses slot c-1 for
its accept test and slot T-1 draws the final token, so a tree whose branching
is all ones consumes exactly the chain's uniforms.
"""
from __future__ import annotations

MASK64 = (1 << 64) - 1
M0 = 0xD2E7470EE14C6C93
M1 = 0xCA5A826395121157
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def _mulhilo(a: int, b: int):
    p = a * b
    return (p >> 64) & MASK64, p & MASK64


def philox4x64(counter, key, rounds: int = ROUNDS):
    """Return the four 64-bit output words for a 4-word counter and 2-word key."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & MASK64
            k1 = (k1 + W1) & MASK64
        hi0, lo0 = _mulhilo(M0, c0)
        hi1, lo1 = _mulhilo(M1, c2)
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform(seed: int, round_: int, b: int, slot: int, tag: int = 0) -> float:
    """The accept/resample uniform for (seed, round, sequence b, slot)."""
    w0 = philox4x64((slot, b, round_, tag), (seed, 0))[0]
    return float(w0 >> 40) * (2.0 ** -24)


class Uniforms:
    """Callable u(b, slot) bound to a (seed, round) pair."""

    def __init__(self, seed: int, round_: int):
        self.seed = int(seed)
        self.round = int(round_)

    def __call__(self, b: int, slot: int) -> float:
        return uniform(self.seed, self.round, b, slot)
