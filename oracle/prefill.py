"""Plain float64 definition of the Qwen3-style batched prefill and the audio head.

Test infrastructure (see the package docstring).  Written as the textbook
decoder layer, one sequence at a time, with no blocking or fusion:

    x = RMS(h; w_in)
    [q | k | v] = x W_qkv^T                     rows of W_qkv: q heads, k heads, v heads
    q_h = RMS(q_h; w_q), k_g = RMS(k_g; w_k)    per head, over head_dim
    q, k <- RoPE(p), p = start_pos + i          rotate-half pairing (m, m + d/2)
    K[slot], V[slot] <- k, v                    slot = cache_slot * capacity + p
    o_h = softmax(q_h K_g^T / sqrt(d) over the visible keys) V_g,  g = h // (Hq/Hkv)
    h <- h + o W_o^T
    x = RMS(h; w_post); [g | u] = x W_gu^T; h <- h + (silu(g) * u) W_down^T

Sources (page title, section):
* "Stabilize Higgs Audio termination and prefill", Summary: the batched prefill
  is embedding lookup, projection GEMMs, q/k norm + RoPE and KV writes.
* flashrt-structures 0.2.0 ``prefill_tower/fp8_chain.py``: the per-call ``run``
  (norm -> merged QKV -> split + RoPE + cache -> attention -> O -> residual ->
  norm -> merged gate/up -> activation -> down -> residual; final fp32 RMSNorm
  times the final weight), ``_build_rope`` (rotate-half: the cosine table is
  duplicated across the two halves of head_dim), ``_prefill_mask_facts`` and the
  module docstring (non-causal attention over exactly the used keys; pads trail
  and their rows are garbage-in-garbage-out), eps 1e-6 (``__init__``).
* "feat(higgs-audio): add checkpoint loading and validation foundation",
  Summary: the final hidden feeds the audio-head projection.

Readings where the pages leave a step open: RMSNorm multiplies by the stored
weight ``w`` (not ``1 + w``); eps 1e-6 for every norm; contiguous GQA groups;
scale 1/sqrt(head_dim); SiLU gate (Qwen3 SwiGLU); RoPE angle
``p * theta**(-2m/d)`` computed in float64.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64


# ------------------------------------------------------------------ elementwise pieces
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """``x * (mean(x^2) + eps)^(-1/2) * w`` over the last axis (fp8_chain ``run``,
    final norm)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def rope_angles(pos: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """phi[i, m] = pos[i] * theta^(-2m/d), m in [0, d/2)."""
    m = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = float(theta) ** (-2.0 * m / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def apply_rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE on x[n, H, d]: pair (m, m + d/2) turns by phi[n, m]."""
    d = x.shape[-1]
    half = d // 2
    phi = rope_angles(pos, d, theta)[:, None, :]
    c, s = np.cos(phi), np.sin(phi)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(scores: np.ndarray) -> np.ndarray:
    """Row softmax with the row max subtracted."""
    z = scores - np.max(scores, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """One head: q[n, d] over keys[j, d] / vals[j, d]; ``visible[i, j]`` masks.

    o[i] = sum_j softmax_j(q_i . k_j / sqrt(d)) v_j over the visible j.
    """
    d = q.shape[-1]
    s = q @ keys.T / np.sqrt(d)
    s = np.where(visible, s, -np.inf)
    return softmax(s) @ vals


# ------------------------------------------------------------------ weights
def widen_layer(bits: dict) -> dict:
    """bf16 bit patterns of one layer -> float64 arrays (exact)."""
    return {k: bf16_to_f64(v) for k, v in bits.items()}


def dense(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x W^T with W stored [out, in]."""
    return x @ w.T


# ------------------------------------------------------------------ one layer
def prefill_layer(m, lw: dict, batch: dict, h: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                  causal: bool = True, used_keys=None, taps: dict | None = None,
                  linear=None) -> np.ndarray:
    """One decoder layer over a packed batch; returns the new residual h[T, D].

    ``m``: model shapes (hidden, n_q_heads, n_kv_heads, head_dim, ffn, rope_theta,
    rms_eps).  ``lw``: float64 weights (``widen_layer``).  ``batch``: ``cu_seqlens``,
    ``start_pos``, ``cache_slot``, ``capacity``.  ``kc``/``vc``: float64 caches
    [n_slots * capacity, Hkv, d], updated in place.  Causal: query i of a
    sequence sees cache positions [0, start_pos + i].  Non-causal: every query
    sees [0, used_keys[s]) and rows i >= used_keys[s] are pads (not written to
    the cache, outputs unspecified).  ``taps`` (optional dict) receives the four
    GEMM inputs (``qkv``, ``o``, ``gu``, ``dn``).  ``linear(site, x, W)`` replaces
    the plain product (used by the FP8 and MXFP4 fake-quant diagnostics).
    """
    D, Hq, Hkv, d = m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim
    F, eps, theta = m.ffn, m.rms_eps, m.rope_theta
    lin = linear or (lambda site, x, w: dense(x, w))
    cu = np.asarray(batch["cu_seqlens"])
    cap = int(batch["capacity"])
    group = Hq // Hkv
    h = np.array(h, dtype=np.float64, copy=True)
    T = h.shape[0]
    x_in = rms_norm(h, lw["in_norm"], eps)
    qkv = lin("qkv", x_in, lw["w_qkv"])
    q = qkv[:, :Hq * d].reshape(T, Hq, d)
    k = qkv[:, Hq * d:(Hq + Hkv) * d].reshape(T, Hkv, d)
    v = qkv[:, (Hq + Hkv) * d:].reshape(T, Hkv, d)
    q = rms_norm(q, lw["q_norm"], eps)
    k = rms_norm(k, lw["k_norm"], eps)
    o = np.zeros((T, Hq, d))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        if n == 0:
            continue
        sp = int(batch["start_pos"][s])
        base = int(batch["cache_slot"][s]) * cap
        pos = sp + np.arange(n)
        qs = apply_rope(q[a:b], pos, theta)
        ks = apply_rope(k[a:b], pos, theta)
        n_write = n if causal else int(used_keys[s])
        kc[base + sp: base + sp + n_write] = ks[:n_write]
        vc[base + sp: base + sp + n_write] = v[a:a + n_write]
        if causal:
            n_keys = sp + n
            visible = np.arange(n_keys)[None, :] <= pos[:, None]
        else:
            n_keys = int(used_keys[s])
            visible = np.ones((n, n_keys), dtype=bool)
        for hh in range(Hq):
            g = hh // group
            o[a:b, hh] = attention(qs[:, hh], kc[base:base + n_keys, g], vc[base:base + n_keys, g], visible)
    o = o.reshape(T, Hq * d)
    h = h + lin("o", o, lw["w_o"])
    x_post = rms_norm(h, lw["post_norm"], eps)
    gu = lin("gu", x_post, lw["w_gu"])
    act = silu(gu[:, :F]) * gu[:, F:]
    h = h + lin("dn", act, lw["w_down"])
    if taps is not None:
        taps.update(qkv=x_in, o=o, gu=x_post, dn=act)
    return h


def new_cache(m, n_slots: int, capacity: int, fill: float = np.nan):
    shape = (n_slots * capacity, m.n_kv_heads, m.head_dim)
    return np.full(shape, fill), np.full(shape, fill)


# ------------------------------------------------------------------ stack + head
def final_norm(m, h: np.ndarray, w_final: np.ndarray) -> np.ndarray:
    """z = RMS(h; w_final) (fp8_chain ``run``, after the last layer)."""
    return rms_norm(h, w_final, m.rms_eps)


def last_rows(batch: dict) -> np.ndarray:
    cu = np.asarray(batch["cu_seqlens"])
    return cu[1:] - 1


def head_logits(z_last: np.ndarray, w_head: np.ndarray, n_codebooks: int, cb_vocab: int) -> np.ndarray:
    """Audio-head projection of the last hidden row of each sequence:
    logits[s, k, v] = z_s . W_head[k * V + v] ("feat(higgs-audio) ...", Summary)."""
    out = dense(z_last, w_head)
    return out.reshape(z_last.shape[0], n_codebooks, cb_vocab)


def prefill_stack(m, layer_source, batch: dict, h0: np.ndarray, caches: list, w_final: np.ndarray,
                  w_head=None, causal: bool = True, used_keys=None, per_layer=None):
    """h0 -> layers 0..L-1 -> final norm -> head on each sequence's last row.

    ``layer_source(l)`` returns layer l's float64 weights (drawn on demand, so a
    36-layer stack never holds all weights at once).  ``caches[l]`` = (kc, vc).
    ``per_layer(l, h)`` (optional) sees each layer's output.  Returns
    (h_L, z, logits or None).
    """
    h = np.asarray(h0, dtype=np.float64)
    for l in range(m.n_layers):
        kc, vc = caches[l]
        h = prefill_layer(m, layer_source(l), batch, h, kc, vc, causal, used_keys)
        if per_layer is not None:
            per_layer(l, h)
    z = final_norm(m, h, w_final)
    logits = None
    if w_head is not None:
        logits = head_logits(z[last_rows(batch)], w_head, m.n_codebooks, m.cb_vocab)
    return h, z, logits
