"""Philox4x64-10 and the uniforms each ISD decision consumes.

The generator is the counter-based Philox4x64 with 10 rounds from Salmon,
Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11),
written here from that definition with Python integers:

* state: four 64-bit counter words (c0, c1, c2, c3) and two key words (k0, k1);
* one round multiplies c0 and c2 by the two published multipliers into 128-bit
  products, then forms (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1,
  lo(c0*M0));
* between rounds the key is bumped by the two Weyl constants (golden ratio and
  sqrt(3) - 1, as 64-bit fractions).

The pages fix no generator, so this is a reading: one Philox block per decided
token, keyed by the 128-bit step seed, with counter
``(request id, absolute position of the decided token, step, 0)``.  Word 0
gives the uniform for the accept test and word 1 the uniform for residual
resampling.  A 64-bit word w becomes a double in [0, 1) as
``(w >> 11) * 2**-53`` (53 random bits, exact in float64).
"""

from __future__ import annotations

MASK64 = (1 << 64) - 1

# Philox4x64 round multipliers and Weyl key increments (SC'11, Table 2 / Sec. 5).
MULT0 = 0xD2E7470EE14C6C93
MULT1 = 0xCA5A826395121157
WEYL0 = 0x9E3779B97F4A7C15
WEYL1 = 0xBB67AE8584CAA73B
ROUNDS = 10


def philox4x64(counter, key, rounds: int = ROUNDS):
    """One Philox4x64 block: four 64-bit output words for a counter and a key."""
    c0, c1, c2, c3 = (int(w) & MASK64 for w in counter)
    k0, k1 = (int(w) & MASK64 for w in key)
    for rnd in range(rounds):
        if rnd > 0:
            k0 = (k0 + WEYL0) & MASK64
            k1 = (k1 + WEYL1) & MASK64
        prod0 = MULT0 * c0
        prod1 = MULT1 * c2
        c0, c1, c2, c3 = ((prod1 >> 64) ^ c1 ^ k0,
                          prod1 & MASK64,
                          (prod0 >> 64) ^ c3 ^ k1,
                          prod0 & MASK64)
    return c0, c1, c2, c3


def unit_double(word: int) -> float:
    """Map a 64-bit word to a double in [0, 1) using its top 53 bits."""
    return float((int(word) & MASK64) >> 11) * (2.0 ** -53)


def decision_counter(req_id: int, position: int, step: int):
    """Counter block for the token at absolute ``position`` of request ``req_id``."""
    if req_id < 0 or position < 0 or step < 0:
        raise ValueError("request id, position and step must be non-negative")
    return (req_id, position, step, 0)


def decision_uniforms(seed, req_id: int, position: int, step: int):
    """(u_accept, u_resample) for one decided token."""
    w = philox4x64(decision_counter(req_id, position, step), seed)
    return unit_double(w[0]), unit_double(w[1])
