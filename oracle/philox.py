"""Philox4x32-10 counter-based generator (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The method draws random numbers twice: the jitter of the stratified samples
("Spatial Intelligence - Part 1: NeRF", Section 2 Code, 6. Hierarchical
sampling, ``stratified_sample``) and the uniforms of the inverse-CDF sampler
(same section, ``sample_pdf``).  The pages use ``torch.rand``, whose stream
cannot be reproduced in a GPU kernel, so both sides implement one published
counter-based generator: Philox4x32 with 10 rounds, from J. Salmon,
M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11, section 3.

One round maps a counter (c0, c1, c2, c3) under a key (k0, k1) to
  (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
with 64-bit products of 32-bit words; between rounds the key is bumped by
the Weyl constants (W0, W1) modulo 2^32.

Stream conventions used by the renderer (key = (seed low word, seed high
word)):
  stream 0  stratified jitter:  counter = (ray lo, sample index, ray hi, 0)
  stream 1  inverse-CDF uniforms: counter = (ray lo, fine index, ray hi, 1)
A uniform is (word0 >> 8) * 2^-24, an exact float32 in [0, 1 - 2^-24].
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

STREAM_JITTER = 0
STREAM_PDF = 1


def philox4x32_10(ctr, key):
    """Apply Philox4x32-10.  ``ctr`` is a tuple of 4 arrays (or ints) of
    32-bit words, ``key`` a tuple of 2; broadcasting applies.  Returns a tuple
    of 4 uint64 arrays holding 32-bit words."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & np.uint64(MASK32) for c in ctr)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & np.uint64(MASK32) for k in key)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    mask = np.uint64(MASK32)
    s32 = np.uint64(32)
    for r in range(10):
        if r > 0:
            k0 = (k0 + np.uint64(W0)) & mask
            k1 = (k1 + np.uint64(W1)) & mask
        p0 = m0 * c0  # < 2^64: exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> s32, p0 & mask
        hi1, lo1 = p1 >> s32, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def seed_key(seed: int):
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return (seed & MASK32, seed >> 32)


def uniform_from_word(w) -> np.ndarray:
    """Top 24 bits of a 32-bit word scaled by 2^-24: exact float32 in [0,1)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def uniforms(seed: int, stream: int, ray_ids, sample_ids) -> np.ndarray:
    """Uniform for each (ray, sample) pair; arrays broadcast."""
    ray = np.asarray(ray_ids, dtype=np.uint64)
    smp = np.asarray(sample_ids, dtype=np.uint64)
    ray, smp = np.broadcast_arrays(ray, smp)
    lo = ray & np.uint64(MASK32)
    hi = ray >> np.uint64(32)
    w0, _, _, _ = philox4x32_10((lo, smp, hi, np.full_like(lo, stream)), seed_key(seed))
    return uniform_from_word(w0)
