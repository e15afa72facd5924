"""The delayed-codebook step with sampling and termination policies, step by step.

Test infrastructure (see the package docstring).

Sources:
* "Stabilize Higgs Audio termination and prefill" (FlashRT pull request 141),
  Summary and Root cause: delayed EOC handling must end a stream whichever
  codebook reports EOC first (the old check only handled the first codebook), and
  a bounded, deterministic stop guard ends streams caught in a stable loop of
  repeated codes in which EOC never comes close to top-1.
* vLLM-Omni pull request 8226 (Higgs Audio v3 streaming on Model Runner V2),
  Purpose and Test Plan: per-request temperature / top-k / top-p sampling with
  seeded exponential noise (the row sampler is ``sampling.sample_row``).

Readings where the pages give no rule (each a line in the design notes):
* End frame.  A stream may carry an end frame e (-1 while open).  Aligned frame
  e is the first frame that is all EOC, so codebook k, which emits aligned frame
  f at step f + k, is forced to EOC at every step t >= e + k.
* Cascade (forced delayed-EOC).  When it is on and the stream is open, a step
  whose codes hold EOC in codebooks k1 < ... < kn sets e = t - kn, the earliest
  aligned frame any of them ended (codebooks below kn are then forced from the
  next step on).
* Stop guard.  With a limit R >= 2, an open stream counts consecutive steps whose
  K codes equal the previous step's (the first step of a run counts 1); when the
  count reaches R the stream gets e = t + 1: codebook 0 emits EOC from the next
  step and the rest follow in the delay pattern.  The guard's state (last codes,
  run) is frozen once e is set.
* When both fire at one step, e is the smaller of the two.
* Code of codebook k at step t, in order: BOS while t < k; EOC once codebook k has
  emitted EOC (sticky); EOC when forced by the end frame; else the row's choice
  (greedy argmax, or the sampled token when the stream's temperature is > 0).
* Done streams, the aligned-frame write and the embedding sum are as in
  ``codebook.codebook_step``.
"""
from __future__ import annotations

import numpy as np

from .codebook import argmax_lowest, embed_sum
from .sampling import row_uniforms, sample_row


def codebook_step_policy(logits, frame, eoc_seen, done, bos_id, eoc_id, cb_embed_f32, aligned=None,
                         max_frames=0, *, temperature=None, top_k=None, top_p=None, seed=None,
                         eoc_cascade=False, repeat_limit=0, end_frame=None, last_codes=None,
                         repeat_run=None, choices=None):
    """One decode step for B streams.

    State arrays (``frame``, ``eoc_seen``, ``done``, ``aligned``, ``end_frame``
    int32[B], ``last_codes`` int32[B, K], ``repeat_run`` int32[B]) are updated in
    place.  ``temperature`` / ``top_k`` / ``top_p`` / ``seed`` are per-stream
    arrays (None: greedy, no top-k, no top-p).  ``choices[b, k] >= 0`` replaces
    the row's own choice (teacher forcing of a row whose float decision was too
    close to call).  Returns (codes int32[B, K], emb bf16 bits [B, D], info) where
    ``info[b][k]`` is the row sampler's info dict for every sampled row.
    """
    B, K, V = logits.shape
    D = cb_embed_f32.shape[1]
    codes = np.empty((B, K), dtype=np.int32)
    emb = np.empty((B, D), dtype=np.uint16)
    info = [[None] * K for _ in range(B)]
    for b in range(B):
        if done[b]:
            c = [eoc_id] * K
        else:
            t = int(frame[b])
            e = int(end_frame[b]) if end_frame is not None else -1
            T = float(temperature[b]) if temperature is not None else 0.0
            tk = int(top_k[b]) if top_k is not None else 0
            tp = float(top_p[b]) if top_p is not None else 1.0
            c = []
            for k in range(K):
                if t < k:
                    ck = bos_id                        # delay fill
                elif eoc_seen[b, k]:
                    ck = eoc_id                        # sticky EOC
                elif e >= 0 and t >= e + k:
                    ck = eoc_id                        # forced by the end frame
                elif choices is not None and choices[b, k] >= 0:
                    ck = int(choices[b, k])
                elif T > 0.0:
                    ck, info[b][k] = sample_row(logits[b, k], T, tk, tp,
                                                row_uniforms(int(seed[b]), t, k, V))
                else:
                    ck = argmax_lowest(logits[b, k])
                if ck == eoc_id:
                    eoc_seen[b, k] = 1
                c.append(ck)
                if aligned is not None and t >= k and t - k < max_frames:
                    aligned[b, t - k, k] = ck
            if e < 0:
                cand = []
                if repeat_limit > 0:
                    run = int(repeat_run[b]) + 1 if [int(v) for v in last_codes[b]] == c else 1
                    repeat_run[b] = run
                    last_codes[b] = c
                    if run >= repeat_limit:
                        cand.append(t + 1)
                if eoc_cascade:
                    ended = [k for k in range(K) if c[k] == eoc_id]
                    if ended:
                        cand.append(t - max(ended))
                if cand:
                    end_frame[b] = min(cand)
            frame[b] = t + 1
            done[b] = 1 if all(eoc_seen[b, k] for k in range(K)) else 0
        codes[b] = c
        emb[b] = embed_sum(cb_embed_f32, c, V)
    return codes, emb, info
