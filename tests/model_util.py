"""Upload seeded model weights to the device and build the C structures the
prefill calls take (test and bench plumbing; no method arithmetic)."""
from __future__ import annotations

import numpy as np

import synth

LAYER_KEYS = ("in_norm", "post_norm", "q_norm", "k_norm", "w_qkv", "w_o", "w_gu", "w_down")


def upload_layer(bits: dict) -> dict:
    from gpu_util import dev_bf16
    return {k: dev_bf16(bits[k]) for k in LAYER_KEYS}


def fp8_pack(H, dl: dict, m) -> tuple:
    """E4M3 weights with per-output-channel scales, packed on the device by
    hr_quantize_weight_e4m3.  Returns (device weights dict, scale dict)."""
    import torch
    out = dict(dl)
    scales = {}
    shapes = {"w_qkv": (m.qkv_rows, m.hidden), "w_o": (m.hidden, m.attn_width),
              "w_gu": (2 * m.ffn, m.hidden), "w_down": (m.hidden, m.ffn)}
    site = {"w_qkv": "qkv", "w_o": "o", "w_gu": "gu", "w_down": "dn"}
    for name, (N, K) in shapes.items():
        w8 = torch.empty((N, K), dtype=torch.uint8, device="cuda")
        sc = torch.empty(N, dtype=torch.float32, device="cuda")
        H.hr_quantize_weight_e4m3(dl[name], N, K, w8, sc)
        out[name] = w8
        scales[site[name]] = sc
    return out, scales


def mx_pack(H, dl: dict, m, awq: dict | None = None) -> tuple:
    """MXFP4 weights of O, gate/up and down packed on the device by
    hr_quantize_mxfp4 (AWQ vectors ``awq`` = {"o", "gu", "dn"} of s; None: 1).
    Returns (device weights dict with the codes in place of w_o / w_gu / w_down,
    the make_layer ``mx`` dict of scales and 1/s vectors)."""
    import torch
    from gpu_util import dev
    D, F, A = m.hidden, m.ffn, m.n_q_heads * m.head_dim
    out = dict(dl)
    mxd = {}
    s = inv = None
    if awq is not None:
        s = {k: np.asarray(v, np.float64).astype(np.float32) for k, v in awq.items()}
        inv = {k: (1.0 / np.asarray(v, np.float64)).astype(np.float32) for k, v in awq.items()}
    row_gu = np.concatenate([np.ones(F, np.float32), inv["dn"]]) if inv is not None else None
    for name, key, N, K, site, row in (("w_o", "o_s", D, A, "o", None), ("w_gu", "gu_s", 2 * F, D, "gu", row_gu),
                                       ("w_down", "down_s", D, F, "dn", None)):
        c = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
        sc = torch.zeros((K // 128) * N * 4, dtype=torch.uint8, device="cuda")
        H.hr_quantize_mxfp4(dl[name], N, K, c, sc, N, col_scale=dev(s[site]) if s is not None else None,
                            row_scale=dev(row) if row is not None else None)
        out[name], mxd[key] = c, sc
    mxd["inv_o"] = dev(inv["o"]) if inv is not None else None
    mxd["inv_gu"] = dev(inv["gu"]) if inv is not None else None
    return out, mxd


def dims_of(H, m, causal=True, n_layers=None):
    return H.make_dims(m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim, m.ffn,
                       n_layers if n_layers is not None else m.n_layers, m.rope_theta, m.rms_eps, causal)


def kv_cache(m, n_slots: int, capacity: int, poison=True):
    import torch
    from gpu_util import poisoned_bf16
    shape = (n_slots * capacity, m.n_kv_heads, m.head_dim)
    if poison:
        return poisoned_bf16(shape), poisoned_bf16(shape)
    return (torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
            torch.zeros(shape, dtype=torch.bfloat16, device="cuda"))


def workspace(H, dims, wtype, T):
    import torch
    return torch.empty(max(1, H.hr_workspace_bytes(dims, wtype, T)), dtype=torch.uint8, device="cuda")


def cu_of(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
