"""Philox-4x32-10 counter-based generator, NumPy uint64 arithmetic.

Definition: Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10 rounds.  One round maps
the counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

where hi/lo are the upper/lower 32 bits of the 64-bit product.  Between rounds
the key is bumped by the Weyl constants (W0, W1) modulo 2^32.  The multipliers
and Weyl constants are the ones the paper gives for the 4x32 variant.

The page "Real-Time Inference for JEPA World Model Architectures with Ray"
(section 01) only says candidates are drawn from a Gaussian; the generator is
fixed by the method's description of the sampler as Philox-4x32.
Pinned in the tests against rocRAND's philox4x32_10 engine (an independent
open-source implementation, compiled on the host).
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter: np.ndarray, key) -> np.ndarray:
    """Apply Philox-4x32-10 to counters.

    counter: uint32 array [..., 4]; key: (k0, k1) 32-bit integers.
    Returns uint32 array [..., 4] of output words (w0, w1, w2, w3).
    """
    c = np.asarray(counter, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = int(key[0]) & 0xFFFFFFFF
    k1 = int(key[1]) & 0xFFFFFFFF
    for rnd in range(ROUNDS):
        if rnd > 0:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = np.uint64(M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed: int):
    """Key of a 64-bit seed: (low 32 bits, high 32 bits)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32
