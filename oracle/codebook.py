"""The delayed-codebook step of a multi-codebook audio head, step by step.

Test infrastructure (see the package docstring).

Source: "Stabilize Higgs Audio termination and prefill" (FlashRT pull request
141), Summary (a shared helper does per-frame argmax, delay handling and
codebook-embedding accumulation; delayed EOC handling is fixed) and Root cause
(the old delayed-EOC check only handled the first codebook reliably).  The delay
pattern itself: codebook k runs k frames behind codebook 0, so at decode step t
codebook k emits the code of aligned frame t - k and is filled with BOS while
t < k; a stream ends only once every codebook has emitted EOC.

Readings where the page is silent (one sentence each):
* BOS = V - 2 and EOC = V - 1 (the last two ids of each codebook vocabulary).
* argmax takes the lowest index among equal maxima.
* EOC is sticky per codebook: once codebook k has emitted EOC it keeps emitting
  EOC.  There is no forced cascade; argmax is not masked (BOS may win at t >= k).
* A stream that is already done emits EOC on every codebook and its state does
  not change; its embedding is still formed from those EOC rows.
* The embedding is the fp32 sum, in codebook order starting from codebook 0's
  row, of the K selected rows of the codebook-embedding table, rounded once to
  bf16 (nearest, ties to even).  This precision is part of the step's contract,
  so this function computes it in float32, not float64.
"""
from __future__ import annotations

import numpy as np

from .numerics import f32_to_bf16


def argmax_lowest(row: np.ndarray) -> int:
    """Index of the largest value; the lowest such index on ties."""
    best = 0
    for j in range(1, row.shape[0]):
        if row[j] > row[best]:
            best = j
    return best


def codebook_step(logits: np.ndarray, frame: np.ndarray, eoc_seen: np.ndarray, done: np.ndarray,
                  bos_id: int, eoc_id: int, cb_embed_f32: np.ndarray, aligned=None,
                  max_frames: int = 0):
    """One decode step for B streams.

    ``logits[B, K, V]`` (any real dtype; compared exactly), ``frame[B]`` int32,
    ``eoc_seen[B, K]`` and ``done[B]`` uint8 are updated in place, as is
    ``aligned[B, max_frames, K]`` (when given): aligned frame f of codebook k is
    written when it is emitted, at step f + k.  ``cb_embed_f32[K * V, D]`` holds
    the codebook-embedding rows.  Returns (codes int32[B, K], emb bf16 bits [B, D]).
    """
    B, K, V = logits.shape
    D = cb_embed_f32.shape[1]
    codes = np.empty((B, K), dtype=np.int32)
    emb = np.empty((B, D), dtype=np.uint16)
    for b in range(B):
        if done[b]:
            c = [eoc_id] * K
        else:
            t = int(frame[b])
            c = []
            for k in range(K):
                if t < k:
                    ck = bos_id                        # delay fill
                elif eoc_seen[b, k]:
                    ck = eoc_id                        # sticky EOC
                else:
                    ck = argmax_lowest(logits[b, k])
                if ck == eoc_id:
                    eoc_seen[b, k] = 1
                c.append(ck)
                if aligned is not None and t >= k and t - k < max_frames:
                    aligned[b, t - k, k] = ck
            frame[b] = t + 1
            done[b] = 1 if all(eoc_seen[b, k] for k in range(K)) else 0
        codes[b] = c
        emb[b] = embed_sum(cb_embed_f32, c, V)
    return codes, emb


def embed_sum(cb_embed_f32: np.ndarray, c, V: int) -> np.ndarray:
    """bf16 bits of the fp32 sum, in codebook order, of rows k * V + c[k]."""
    acc = cb_embed_f32[0 * V + c[0]].astype(np.float32).copy()
    for k in range(1, len(c)):
        acc = (acc + cb_embed_f32[k * V + c[k]].astype(np.float32)).astype(np.float32)
    return f32_to_bf16(acc)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Largest minus second-largest value of each row (float64)."""
    x = np.sort(np.asarray(logits, dtype=np.float64), axis=-1)
    return x[..., -1] - x[..., -2]
