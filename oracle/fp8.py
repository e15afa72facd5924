"""Static FP8 (E4M3) prefill: weight scales, activation calibration, fake-quant layer.

Test infrastructure (see the package docstring).

Source: flashrt-structures 0.2.0 ``prefill_tower/fp8_chain.py``:
* the quantiser table (``_quantize``): each of the four GEMM sites of a layer
  (qkv, o, gu, dn) gets a static per-tensor activation scale ``amax / FP8_MAX``
  and the GEMM runs with ``alpha = activation scale x weight scale``;
* the calibration probe: forward pre-hooks record the peak |activation| at each
  site's input on a probe prompt; one sample's raw maximum is the statistic
  (quantile 1.0); a site whose peak is not positive refuses the bind;
* "Stabilize Higgs Audio termination and prefill", Summary / Root cause: the
  calibration prompt is a fixed built-in prompt, not the first user request.

Readings where the pages leave a step open:
* weight scales are per output channel: ``s_w[n] = max_k |W[n, k]| / 448`` and
  the stored weight is ``e4m3(W[n, k] / s_w[n])``; the division and the scale
  are float32 (the precision the packed weight is produced in), so the codes
  are a bit-exact contract;
* the quantised activation is the tensor the GEMM consumes (the norm output
  including its weight, the attention output, the SwiGLU product);
* attention itself (q, k, v, softmax) stays in high precision.
"""
from __future__ import annotations

import numpy as np

from .numerics import E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_round
from .prefill import prefill_layer

SITES = ("qkv", "o", "gu", "dn")


def weight_scales_e4m3(w_f32: np.ndarray):
    """Per-output-channel scale and E4M3 codes of W[N, K] (float32 arithmetic)."""
    w = np.asarray(w_f32, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = (w / s[:, None]).astype(np.float32)
    return s, e4m3_encode(q)


def calibrate(m, lw: dict, h0: np.ndarray, capacity: int | None = None) -> dict:
    """Static activation scales of one layer from one calibration prompt.

    Runs the float64 layer non-causally over all rows of ``h0`` (every key used),
    takes the raw peak |x| at the four GEMM inputs and returns
    ``{site: amax / 448}``.  Raises if a site's peak is not positive.
    """
    n = h0.shape[0]
    cap = capacity or n
    batch = {"cu_seqlens": np.array([0, n]), "start_pos": np.array([0]),
             "cache_slot": np.array([0]), "capacity": cap}
    kc = np.zeros((cap, m.n_kv_heads, m.head_dim))
    vc = np.zeros_like(kc)
    taps: dict = {}
    prefill_layer(m, lw, batch, h0, kc, vc, causal=False, used_keys=[n], taps=taps)
    scales = {}
    for site in SITES:
        amax = float(np.max(np.abs(taps[site])))
        if not amax > 0.0:
            raise ValueError(f"dead quantizer site {site}: amax={amax}")
        scales[site] = amax / E4M3_MAX
    return scales


def fake_quant_linear(scales: dict, packed: dict):
    """``linear(site, x, W)`` computing a * s_w[n] * sum_k e4m3(x/a)[m, k] W8[n, k]."""
    def lin(site, x, _w):
        a = scales[site]
        s_w, codes = packed[site]
        xq = e4m3_round(np.asarray(x, dtype=np.float64) / a)
        return (xq @ e4m3_decode(codes).T) * (a * s_w.astype(np.float64))[None, :]
    return lin


def fp8_layer(m, lw: dict, scales: dict, packed: dict, batch: dict, h, kc, vc,
              causal: bool, used_keys=None) -> np.ndarray:
    """The layer with the four GEMMs run on E4M3 operands (a diagnostic of what
    the FP8 chain computes; the pass criterion compares against the unquantised
    layer)."""
    return prefill_layer(m, lw, batch, h, kc, vc, causal, used_keys,
                         linear=fake_quant_linear(scales, packed))


def pack_layer(lw_f32: dict) -> dict:
    """{site: (s_w, codes)} for the four weight matrices of a layer."""
    names = {"qkv": "w_qkv", "o": "w_o", "gu": "w_gu", "dn": "w_down"}
    return {site: weight_scales_e4m3(lw_f32[names[site]]) for site in SITES}
