"""MXFP4 (OCP Microscaling FP4) for the O and FFN projections, with an AWQ pre-scale.

Test infrastructure (see the package docstring).

Source: flashrt-structures 0.2.0, ``prefill_tower/fp8_chain.py``: the FP4 band
table (the FFN pair and the attention output projection in 4-bit with dynamic
block scales, QKV left as it is), ``_awq_scale`` (per-input-channel pre-scale
s = (a / mean a)^alpha clamped to [0.25, 4], alpha 0.8 in the band table; the
GEMM columns carry s and the tensor feeding the GEMM carries 1/s) and
``_interleave_gu_rows`` (the down projection's 1/s folded into the up rows so a
single gate/up GEMM emits the down GEMM's quantised input).  The pages use
NVIDIA's NVFP4 (16-element blocks, e4m3 scales); gfx950's matrix cores take the
OCP MX form natively, which this module follows:

* FP4 E2M1 (OCP MX specification v1.0, element formats): 1 sign bit, 2 exponent
  bits with bias 1, 1 mantissa bit; exponent 0 holds 0 and 0.5; magnitudes
  0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.  Encoding rounds to nearest,
  ties to the even code, and saturates at 6.
* Block scaling (same specification, conversion of a block): blocks of 32
  consecutive values along K share an E8M0 scale X = 2^e (a biased-127
  exponent byte), e = floor(log2(max |v|)) - 2 (2 = the exponent of E2M1's
  largest normal), clamped to [-127, 127]; each value is encoded as v / X.  An
  all-zero block takes the byte 0.

Readings (each a line in the design notes): the block runs along the reduction
dimension K for weights and activations alike; activations are quantised per
row at run time (dynamic scales); the weights are packed once, w' = (w * s_col)
* s_row in binary32 (s_col = the AWQ scale of the input channel, s_row = 1 / s
of the down projection for the up rows, else 1); the attention output and the
FFN input carry their 1/s before they are quantised; everything else is float64.
"""
from __future__ import annotations

import numpy as np

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code) -> np.ndarray:
    """Value of 4-bit codes, from the field layout (sign | exponent(2) | mantissa(1))."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.power(2.0, e - 1))
    return sign * mag


def e2m1_encode(x) -> np.ndarray:
    """Nearest code (ties to the even code, i.e. mantissa bit 0), saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    d = np.abs(a[..., None] - E2M1_MAG)                     # distance to each magnitude
    best = np.argmin(d, axis=-1)                           # first (lower) magnitude on a tie
    # a tie between magnitudes j and j+1: take the one with an even code
    tie = np.take_along_axis(d, np.minimum(best + 1, 7)[..., None], -1)[..., 0] == \
        np.take_along_axis(d, best[..., None], -1)[..., 0]
    tie &= best < 7
    best = np.where(tie & (best % 2 == 1), best + 1, best)
    best = np.where(a > 6.0, 7, best)
    return np.where(np.signbit(x) & (best > 0), best | 8, best).astype(np.uint8)


def block_scale_exp(amax) -> np.ndarray:
    """Shared exponent e of blocks with the given max |v|: floor(log2 amax) - 2,
    clamped to [-127, 127]; -127 for an all-zero block."""
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    # floor(log2 a) from the binade, exact for every binary64 value
    _, ex = np.frexp(safe)                                  # safe = m * 2^ex, m in [0.5, 1)
    e = ex.astype(np.int64) - 1 - 2
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127)


def quantize_blocks(v: np.ndarray):
    """MX block quantisation along the last axis (a multiple of 32).

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K / 32]); the scale
    byte is e + 127.
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    assert K % 32 == 0
    blk = v.reshape(*v.shape[:-1], K // 32, 32)
    e = block_scale_exp(np.max(np.abs(blk), axis=-1))
    codes = e2m1_encode(blk / np.power(2.0, e)[..., None])
    return codes.reshape(v.shape), (e + 127).astype(np.uint8)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    K = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(*codes.shape[:-1], K // 32, 32)
    X = np.power(2.0, scales.astype(np.int64) - 127)
    return (vals * X[..., None]).reshape(codes.shape)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def awq_scale(chan_amax: np.ndarray, alpha: float = 0.8) -> np.ndarray:
    """Per-input-channel pre-scale: (a / mean a)^alpha, a >= 1e-6, clamped to [0.25, 4]."""
    a = np.maximum(np.asarray(chan_amax, dtype=np.float64), 1e-6)
    return np.clip(np.power(a / a.mean(), alpha), 0.25, 4.0)


def pack_weight(w_bf16_f32: np.ndarray, col_scale=None, row_scale=None):
    """Weight packing: w' = (w * s_col) * s_row in binary32, then MX blocks.

    ``w_bf16_f32`` holds the bf16 weights widened to float32 [N, K]; the scales
    are float32 vectors.  Returns (codes uint8 [N, K], scale bytes [N, K / 32]).
    """
    w = np.asarray(w_bf16_f32, dtype=np.float32)
    if col_scale is not None:
        w = (w * np.asarray(col_scale, np.float32)[None, :]).astype(np.float32)
    if row_scale is not None:
        w = (w * np.asarray(row_scale, np.float32)[:, None]).astype(np.float32)
    return quantize_blocks(w.astype(np.float64))


def mx_matmul(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """y[m, n] = sum_k A[m, k] B[n, k] of the dequantised blocks (float64)."""
    return dequantize_blocks(a_codes, a_scales) @ dequantize_blocks(b_codes, b_scales).T


# ------------------------------------------------------------------ the MXFP4 band of a layer
SITES = ("o", "gu", "dn")


def calibrate_awq(m, lw: dict, h0: np.ndarray, alpha: float = 0.8) -> dict:
    """AWQ pre-scales {site: s} from the per-input-channel peak |x| at the O,
    gate/up and down inputs of the float64 layer on one calibration prompt (run
    non-causally over all its rows, as the FP8 calibration)."""
    from .prefill import prefill_layer
    n = h0.shape[0]
    batch = {"cu_seqlens": np.array([0, n]), "start_pos": np.array([0]), "cache_slot": np.array([0]),
             "capacity": n}
    kc = np.zeros((n, m.n_kv_heads, m.head_dim))
    vc = np.zeros_like(kc)
    taps: dict = {}
    prefill_layer(m, lw, batch, h0, kc, vc, causal=False, used_keys=[n], taps=taps)
    return {site: awq_scale(np.max(np.abs(taps[site]), axis=0), alpha) for site in SITES}


def pack_layer(lw_f32: dict, awq: dict) -> dict:
    """Packed MXFP4 weights {site: (codes [N, K], scale bytes [N, K / 32])} and
    the binary32 vectors the packing and the activations use.

    O: columns times s_o.  gate/up: columns times s_gu, and the up rows (F..2F)
    times 1 / s_dn.  down: columns times s_dn.  The activations take 1 / s_o
    (attention output) and 1 / s_gu (FFN input); the down input already carries
    1 / s_dn through the up rows.
    """
    F = lw_f32["w_down"].shape[1]
    s = {k: np.asarray(v, np.float64).astype(np.float32) for k, v in awq.items()}
    inv = {k: (1.0 / np.asarray(v, np.float64)).astype(np.float32) for k, v in awq.items()}
    row_gu = np.concatenate([np.ones(F, np.float32), inv["dn"]])
    packed = {"o": pack_weight(lw_f32["w_o"], s["o"]),
              "gu": pack_weight(lw_f32["w_gu"], s["gu"], row_gu),
              "dn": pack_weight(lw_f32["w_down"], s["dn"])}
    return {"packed": packed, "col": s, "inv": inv, "row_gu": row_gu}


def mx_linear(pk: dict):
    """``linear(site, x, W)`` for ``prefill.prefill_layer``: QKV as it is; O and
    gate/up inputs times their 1/s, then every MXFP4 site quantises its input in
    blocks of 32 and multiplies the packed weight."""
    from .prefill import dense

    def lin(site, x, w):
        if site == "qkv":
            return dense(x, w)
        x = np.asarray(x, dtype=np.float64)
        if site in ("o", "gu"):
            x = x * pk["inv"][site].astype(np.float64)[None, :]
        codes, sc = quantize_blocks(x)
        wc, ws = pk["packed"][site]
        return mx_matmul(codes, sc, wc, ws)
    return lin


def mx_layer(m, lw: dict, pk: dict, batch: dict, h, kc, vc, causal: bool = True, used_keys=None) -> np.ndarray:
    """The layer with O, gate/up and down on MXFP4 operands (QKV and attention
    unchanged): each GEMM input is quantised from its full-precision value."""
    from .prefill import prefill_layer
    return prefill_layer(m, lw, batch, h, kc, vc, causal, used_keys, linear=mx_linear(pk))
