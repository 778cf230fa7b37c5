"""Plain CPU oracle of inverted dropout with masks drawn by a counter-based
generator.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the GPU library.

Sources (page title, section):
  * Hephaistos, "Architecture at a glance": inverted dropout on the
    embeddings, the attention weights and the attention and MLP outputs;
    "Design notes": masks are sampled only by the training forward and reused
    by its paired backward.
  * randyGPT, "Architecture Details": dropout after the attention projection
    and the MLP output, training only; "Default hyperparameters": 0.1.

Readings (the pages name the sites and the rate, nothing more):
  * Sites built: 0 = the embedding output, 1 = the attention projection's
    output (the parallel block: its one combined attention + MLP projection),
    2 = the MLP output (Llama block), each before its residual add, and 3 =
    the attention weights: the softmax probabilities p_ij of head h of
    sequence b are multiplied by the mask of element ((b H + h) T + i) T + j
    of a [B H T, T] tensor before they weight the values (the softmax
    normaliser is taken before dropout).
  * Inverted dropout: a kept element is multiplied by 1/(1-p) (that factor
    rounded once to float32, as the GPU applies it), a dropped one is 0.
  * Masks come from Philox-4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
    random numbers: as easy as 1, 2, 3", SC 2011), implemented here from its
    published definition.  Element e of a site's [tokens, C] tensor (e = row
    C + column) takes word e mod 4 of the generator's output for the counter
    (q mod 2^32, q div 2^32, site, layer), q = e div 4, under the key
    (seed mod 2^32, seed div 2^32); it is kept iff that word is at least
    floor(p 2^32).  The backward regenerates the same masks from the same
    counters, which is the pages' "reuse".
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "dropout_multiplier"]

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)   # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85                          # key schedule (Weyl) increments
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox-4x32-10 on arrays: ctr = (c0, c1, c2, c3) of uint32 arrays (or
    scalars), key = (k0, k1) ints.  Ten rounds; in each, the two 32x32->64
    products of c0 and c2 with the round multipliers give the new words
    (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)), then
    the key is bumped by the Weyl increments (mod 2^32)."""
    c0, c1, c2, c3 = (np.asarray(c, np.uint64) & _LO for c in ctr)
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = c0 * _M0
        p1 = c2 * _M1
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & _LO,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & _LO)
        k0 = (k0 + _W0) & 0xFFFFFFFF
        k1 = (k1 + _W1) & 0xFFFFFFFF
    return tuple(np.asarray(c, np.uint64).astype(np.uint32) for c in (c0, c1, c2, c3))


def dropout_multiplier(p, seed, site, layer, rows, C):
    """The [rows, C] float64 array of multipliers of one dropout site: 0 for a
    dropped element, float32(1/(1-p)) for a kept one (see the module readings
    for the mask).  p = 0 gives all ones."""
    if p <= 0.0:
        return np.ones((rows, C))
    e = np.arange(rows * C, dtype=np.uint64)
    q = e >> np.uint64(2)
    words = philox4x32_10((q & _LO, q >> np.uint64(32), np.full_like(q, site), np.full_like(q, layer)),
                          (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    w = (e & np.uint64(3)).astype(np.int64)
    r = np.choose(w, words)
    thr = np.uint64(int(np.floor(p * 4294967296.0)))
    keep = r.astype(np.uint64) >= thr
    scale = float(np.float32(1.0 / (1.0 - p)))
    return np.where(keep, scale, 0.0).reshape(rows, C)
