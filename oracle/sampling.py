"""Seeded sampling of one codebook row: temperature, top-k, top-p, exponential race.

Test infrastructure (see the package docstring).

Source: vLLM-Omni pull request 8226 (Higgs Audio v3 streaming on Model Runner
V2).  Purpose: the model's own delayed-codebook sampler supports temperature,
top-k and top-p, and draws per-request seeded exponential noise for every row;
Test Plan: the serving runs use temperature 1, top-k 50, top-p 0.95; "Step-overhead
reductions": the noise of every request comes from that request's own seeded
generator, in one launch for all requests.

The page names the parts, not the arithmetic that joins them.  Readings (each a
line in the design notes):
* The noise generator is Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011): key = (seed, 0); the counter of
  row k of stream b at step t is (t, k, v // 4, 0), and element v takes word
  v % 4 of that block.  A word x gives u = (floor(x / 2**41) + 1/2) / 2**23, a
  point in (0, 1) that binary32 represents exactly, and the exponential draw
  E = -ln(u).
* Temperature T > 0 divides the logits: z = x / T.  T <= 0 means greedy (the
  lowest-index argmax of the logits), with no noise.
* top-k keeps every element whose logit is at least the k-th largest logit (all
  elements tied with it stay); k <= 0 or k >= V turns it off.  The ranking uses
  the logits themselves: a positive temperature does not change it.
* top-p orders the top-k survivors by logit, larger first, equal logits by lower
  index, and keeps an element when the probability mass of the survivors ahead
  of it (softmax of z over the top-k survivors) is below p: the shortest prefix
  whose mass reaches p.  p >= 1 turns it off; p <= 0 keeps only the first
  element of that order (the limit p -> 0).
* The race: among the kept elements the winner maximises p_v / E_v, i.e.
  z_v - ln(E_v); equal scores go to the lower index.  With independent Exp(1)
  draws the winner is distributed as the renormalised probabilities.

Everything here is float64, with plain Python integers or exact uint64 NumPy
arithmetic for the generator.
"""
from __future__ import annotations

import numpy as np

from .codebook import argmax_lowest

# Philox4x64 multipliers and Weyl key increments (the paper's Table of
# constants for the 4x64 variant)
_M0 = 0xD2E7470EE14C6C93
_M1 = 0xCA5A826395121157
_W0 = 0x9E3779B97F4A7C15
_W1 = 0xBB67AE8584CAA73B
_MASK64 = (1 << 64) - 1
_U32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: int, b: np.ndarray):
    """(high, low) 64-bit halves of the 128-bit product a * b, exactly."""
    a = np.uint64(a)
    a0, a1 = a & _U32, a >> _S32
    b0, b1 = b & _U32, b >> _S32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1    # each < 2**64
    mid = (p00 >> _S32) + (p01 & _U32) + (p10 & _U32)           # < 3 * 2**32
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = (p00 & _U32) | ((mid & _U32) << _S32)
    return hi, lo


def philox4x64(counter, key):
    """Philox4x64-10 of counter blocks (4 uint64 arrays) under key (2 ints).

    Ten rounds; the key gets its Weyl increment before every round after the
    first.  A round multiplies words 0 and 2 by the two constants and mixes the
    high halves with words 1 and 3 and the key.  Returns the 4 output words.
    """
    c = [np.asarray(w, dtype=np.uint64).copy() for w in counter]
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    for r in range(10):
        if r:
            k0, k1 = (k0 + _W0) & _MASK64, (k1 + _W1) & _MASK64
        h0, l0 = _mulhilo(_M0, c[0])
        h1, l1 = _mulhilo(_M1, c[2])
        c = [h1 ^ c[1] ^ np.uint64(k0), l1, h0 ^ c[3] ^ np.uint64(k1), l0]
    return c


def uniform_from_word(x: np.ndarray) -> np.ndarray:
    """u = (top 23 bits of x + 1/2) / 2**23, in (0, 1), as float64 (exact)."""
    top = (np.asarray(x, dtype=np.uint64) >> np.uint64(41)).astype(np.float64)
    return (top + 0.5) / float(1 << 23)


def row_uniforms(seed: int, step: int, k: int, V: int) -> np.ndarray:
    """The V uniforms of codebook row k of a stream with this seed at this step."""
    nb = (V + 3) // 4
    blk = np.arange(nb, dtype=np.uint64)
    z = np.zeros(nb, dtype=np.uint64)
    words = philox4x64([np.full(nb, step, dtype=np.uint64), np.full(nb, k, dtype=np.uint64), blk, z],
                       (seed, 0))
    w = np.stack(words, axis=1).reshape(-1)[:V]     # element v = word v % 4 of block v // 4
    return uniform_from_word(w)


def sample_row(x: np.ndarray, temperature: float, top_k: int, top_p: float, u: np.ndarray):
    """One row's choice.

    ``x`` holds the V logits (any real dtype, widened exactly), ``u`` the row's
    V uniforms.  Returns ``(choice, info)``; ``info`` has the kept set and two
    margins that say how close a float decision came: ``p_margin``, the smallest
    |mass ahead - p * S| over the top-k survivors relative to S (top-p membership),
    and ``race_margin``, the winner's score minus the best other kept score.
    """
    x = np.asarray(x, dtype=np.float64)
    V = x.shape[0]
    info = {"kept": None, "p_margin": np.inf, "race_margin": np.inf, "scores": None}
    if temperature <= 0.0:
        c = argmax_lowest(x)
        info["kept"] = np.array([c])
        return c, info
    # top-k: at least the k-th largest logit
    if 0 < top_k < V:
        kth = np.sort(x)[::-1][top_k - 1]
        in_k = x >= kth
    else:
        in_k = np.ones(V, dtype=bool)
    z = x / float(temperature)
    zmax = z[in_k].max()
    q = np.where(in_k, np.exp(z - zmax), 0.0)
    S = q.sum()
    kept = in_k.copy()
    if top_p < 1.0:
        order = sorted(np.nonzero(in_k)[0], key=lambda v: (-x[v], v))
        kept[:] = False
        ahead = 0.0
        margin = np.inf
        for n, v in enumerate(order):
            if top_p <= 0.0:
                keep = n == 0
            else:
                keep = ahead < top_p * S
                margin = min(margin, abs(ahead - top_p * S) / S)
            kept[v] = keep
            ahead += q[v]
        info["p_margin"] = margin
    E = -np.log(np.asarray(u, dtype=np.float64))
    score = np.where(kept, z - np.log(E), -np.inf)
    c = argmax_lowest(score)
    others = np.delete(score, c)
    info["race_margin"] = score[c] - (others.max() if others.size else -np.inf)
    info["kept"] = np.nonzero(kept)[0]
    info["scores"] = score
    return c, info


def relaxed_kept(x: np.ndarray, temperature: float, top_k: int, top_p: float, tol: float):
    """Kept sets with the top-p bar moved by +tol * S (wide) and -tol * S (narrow).

    Only the top-p test compares floats; for 0 < p < 1 a choice that a float32
    computation could make lies in the wide set.  Returns (wide, narrow) masks.
    """
    x = np.asarray(x, dtype=np.float64)
    V = x.shape[0]
    if 0 < top_k < V:
        in_k = x >= np.sort(x)[::-1][top_k - 1]
    else:
        in_k = np.ones(V, dtype=bool)
    if temperature <= 0.0:
        g = np.arange(V) == argmax_lowest(x)
        return g, g
    order = sorted(np.nonzero(in_k)[0], key=lambda v: (-x[v], v))
    if top_p >= 1.0:
        return in_k, in_k
    if top_p <= 0.0:
        g = np.arange(V) == order[0]
        return g, g
    z = x / float(temperature)
    q = np.where(in_k, np.exp(z - z[in_k].max()), 0.0)
    S = q.sum()
    wide = np.zeros(V, dtype=bool)
    narrow = np.zeros(V, dtype=bool)
    ahead = 0.0
    for v in order:
        wide[v] = ahead < top_p * S + tol * S
        narrow[v] = ahead < top_p * S - tol * S
        ahead += q[v]
    return wide, narrow
