"""ctypes binding of libhr (include/hr.h, include/hr_ops.h).

Argument marshalling only: every step of the path runs in libhr's HIP kernels.
Torch tensors are used for device memory and streams; their data pointers and
the current HIP stream are handed to the C functions of the same names.  A
missing libhr.so raises immediately (there is no fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# HR_LIB selects another build of the same library (the host-sanitizer build)
LIB_PATH = os.environ.get("HR_LIB") or os.path.join(_HERE, "libhr.so")

HR_OK, HR_EINVAL, HR_EUNSUPPORTED, HR_ECAPACITY = 0, -1, -2, -3
HR_EBOUND, HR_EWORKSPACE, HR_EALIGN, HR_EHIP = -4, -5, -6, -7
HR_BF16, HR_FP8_E4M3, HR_MXFP4, HR_F16, HR_F16_PACKED = 0, 1, 2, 3, 4
HR_EPI_F32, HR_EPI_RESIDUAL, HR_EPI_SWIGLU = 0, 1, 2
MX_SRC_BF16, MX_SRC_F32, MX_SRC_F16 = 0, 1, 2
STATUS_NAMES = {0: "HR_OK", -1: "HR_EINVAL", -2: "HR_EUNSUPPORTED", -3: "HR_ECAPACITY",
                -4: "HR_EBOUND", -5: "HR_EWORKSPACE", -6: "HR_EALIGN", -7: "HR_EHIP"}

c_i32, c_f32, c_vp, c_sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
P_i32 = ctypes.POINTER(ctypes.c_int32)


class HrDims(ctypes.Structure):
    _fields_ = [("hidden", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32), ("head_dim", c_i32),
                ("ffn", c_i32), ("n_layers", c_i32), ("rope_theta", c_f32), ("rms_eps", c_f32),
                ("causal", c_i32)]


class HrLayer(ctypes.Structure):
    _fields_ = [("wtype", c_i32),
                ("in_norm_w", c_vp), ("post_norm_w", c_vp), ("q_norm_w", c_vp), ("k_norm_w", c_vp),
                ("w_qkv", c_vp), ("w_o", c_vp), ("w_gu", c_vp), ("w_down", c_vp),
                ("ws_qkv", c_vp), ("ws_o", c_vp), ("ws_gu", c_vp), ("ws_down", c_vp),
                ("as_qkv", c_f32), ("as_o", c_f32), ("as_gu", c_f32), ("as_down", c_f32),
                ("mx_o_s", c_vp), ("mx_gu_s", c_vp), ("mx_down_s", c_vp), ("awq_inv_o", c_vp),
                ("awq_inv_gu", c_vp)]


class HrKv(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("capacity", c_i32), ("n_slots", c_i32)]


class HrBatch(ctypes.Structure):
    _fields_ = [("n_seq", c_i32), ("total_tokens", c_i32), ("max_seqlen", c_i32),
                ("cu_seqlens", c_vp), ("start_pos", c_vp), ("cache_slot", c_vp), ("used_keys", c_vp),
                ("h_cu_seqlens", c_vp), ("h_start_pos", c_vp), ("h_cache_slot", c_vp),
                ("h_used_keys", c_vp)]


class HrStepPolicy(ctypes.Structure):
    _fields_ = [("temperature", c_vp), ("top_k", c_vp), ("top_p", c_vp), ("seed", c_vp),
                ("eoc_cascade", c_i32), ("repeat_limit", c_i32), ("end_frame", c_vp),
                ("last_codes", c_vp), ("repeat_run", c_vp)]


class HrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m codebook_decode_amd.build`")
        # torch brings its own HIP runtime; load it first so that libhr's
        # libamdhip64 dependency resolves to that same runtime (one runtime per
        # process: tensors, streams and launches must share it).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        _check_single_hip_runtime()
        P = ctypes.POINTER
        sig = {
            "hr_last_error": (ctypes.c_char_p, []),
            "hr_workspace_bytes": (c_sz, [P(HrDims), c_i32, c_i32]),
            "hr_prefill_layer": (c_i32, [P(HrDims), P(HrLayer), P(HrBatch), c_vp, P(HrKv), c_vp, c_sz, c_vp]),
            "hr_prefill_stack": (c_i32, [P(HrDims), P(HrLayer), P(HrBatch), c_vp, c_vp, c_i32, c_vp, P(HrKv),
                                         c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_vp, c_sz, c_vp]),
            "hr_codebook_step": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                         c_vp, c_vp, c_i32, c_vp, c_i32, c_vp, c_vp]),
            "hr_codebook_step_policy": (c_i32, [c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp,
                                                c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_vp, P(HrStepPolicy),
                                                c_vp]),
            "hr_decode_workspace_bytes": (c_sz, [P(HrDims), c_i32, c_i32]),
            "hr_decode_noalloc_scratch_bytes": (c_sz, []),
            "hr_decode_step_noalloc": (c_i32, [P(HrDims), P(HrLayer), P(HrBatch), c_vp, P(HrKv), c_vp, c_vp, c_i32,
                                               c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp,
                                               c_vp, c_vp]),
            "hr_decode_step": (c_i32, [P(HrDims), P(HrLayer), P(HrBatch), c_vp, P(HrKv), c_vp, c_vp, c_i32, c_i32,
                                       c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp,
                                       c_sz, c_vp]),
            "hr_embed_rmsnorm": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp,
                                         c_i32, c_f32, c_vp]),
            "hr_rmsnorm": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_i32, c_f32, c_vp]),
            "hr_linear_workspace_bytes": (c_sz, [c_i32, c_i32, c_i32, c_i32, c_i32]),
            "hr_pack_weight": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
            "hr_linear": (c_i32, [c_vp, c_vp, c_vp, c_f32, c_i32, c_i32, c_i32, c_i32, c_i32, c_vp, c_f32, c_vp, c_sz,
                                  c_vp]),
            "hr_residual_rmsnorm": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_f32, c_vp, c_i32, c_f32, c_vp]),
            "hr_qknorm_rope_kv": (c_i32, [P(HrDims), P(HrBatch), c_vp, c_vp, c_vp, c_vp, P(HrKv), c_vp]),
            "hr_attention": (c_i32, [P(HrDims), P(HrBatch), c_vp, P(HrKv), c_vp, c_i32, c_f32, c_vp]),
            "hr_attention_f16": (c_i32, [P(HrDims), P(HrBatch), c_vp, c_vp, c_vp, c_i32, c_vp, c_i32, c_f32, c_vp]),
            "hr_qknorm_rope_attention": (c_i32, [P(HrDims), P(HrBatch), c_vp, c_vp, c_vp, P(HrKv), c_vp, c_i32,
                                                 c_f32, c_vp]),
            "hr_attention_chunked_workspace_bytes": (c_sz, [P(HrDims), c_i32, c_i32]),
            "hr_attention_chunked": (c_i32, [P(HrDims), P(HrBatch), c_vp, P(HrKv), c_vp, c_i32, c_f32, c_i32,
                                             c_i32, c_vp, c_sz, c_vp]),
            "hr_head_workspace_bytes": (c_sz, [c_i32, c_i32]),
            "hr_head_logits": (c_i32, [c_vp, P(HrBatch), c_i32, c_vp, c_f32, c_vp, c_i32, c_i32, c_vp, c_vp,
                                       c_sz, c_vp]),
            "hr_quantize_weight_e4m3": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_vp, c_vp]),
            "hr_quantize_mxfp4": (c_i32, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
            "hr_rmsnorm_mxfp4": (c_i32, [c_vp, c_i32, c_i32, c_vp, c_f32, c_vp, c_vp, c_vp, c_i32, c_vp]),
            "hr_linear_mxfp4": (c_i32, [c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp,
                                        c_i32, c_vp, c_sz, c_vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check_single_hip_runtime() -> None:
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    if len(libs) > 1:
        raise RuntimeError(f"two HIP runtimes are loaded in this process: {sorted(libs)}")


# ---------------------------------------------------------------------------- marshalling helpers
def ptr(t) -> int | None:
    """Device (or host) address of a torch tensor / numpy array, None for None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int) -> None:
    if status != HR_OK:
        raise HrError(status, hr_last_error())


def hr_last_error() -> str:
    return lib().hr_last_error().decode()


def make_dims(hidden, n_q_heads, n_kv_heads, head_dim, ffn, n_layers=1, rope_theta=1e6, rms_eps=1e-6,
              causal=True) -> HrDims:
    return HrDims(hidden, n_q_heads, n_kv_heads, head_dim, ffn, n_layers, rope_theta, rms_eps, int(causal))


class Batch:
    """A packed varlen batch: device int32 tensors plus their host mirrors
    (both kept alive here for the C call)."""

    def __init__(self, cu_seqlens, start_pos, cache_slot, used_keys=None, max_seqlen=None, device="cuda"):
        import torch
        self.h_cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        self.h_sp = np.ascontiguousarray(start_pos, dtype=np.int32)
        self.h_slot = np.ascontiguousarray(cache_slot, dtype=np.int32)
        self.h_used = None if used_keys is None else np.ascontiguousarray(used_keys, dtype=np.int32)
        dev = lambda a: None if a is None else torch.from_numpy(a.copy()).to(device)
        self.d_cu, self.d_sp, self.d_slot, self.d_used = (dev(self.h_cu), dev(self.h_sp), dev(self.h_slot),
                                                          dev(self.h_used))
        n = self.h_sp.size
        lens = np.diff(self.h_cu)
        self.c = HrBatch(n, int(self.h_cu[-1]), int(max_seqlen if max_seqlen is not None else
                                                    (lens.max() if n else 0)),
                         ptr(self.d_cu), ptr(self.d_sp), ptr(self.d_slot), ptr(self.d_used),
                         ptr(self.h_cu), ptr(self.h_sp), ptr(self.h_slot), ptr(self.h_used))

    @property
    def total_tokens(self) -> int:
        return int(self.h_cu[-1])


def make_kv(k, v, capacity: int, n_slots: int) -> HrKv:
    kv = HrKv(ptr(k), ptr(v), capacity, n_slots)
    kv._tensors = (k, v)          # the struct holds raw pointers: keep the caches alive with it
    return kv


def make_layer(t: dict, wtype: int = HR_BF16, scales: dict | None = None, wscales: dict | None = None,
               mx: dict | None = None) -> HrLayer:
    """``t``: device tensors in_norm, post_norm, q_norm, k_norm, w_qkv, w_o, w_gu, w_down.
    MXFP4: ``t`` holds the packed codes of w_o / w_gu / w_down and ``mx`` their
    scales (``o_s``, ``gu_s``, ``down_s``) and the 1/s vectors (``inv_o``, ``inv_gu``)."""
    L = HrLayer()
    L.wtype = wtype
    L.in_norm_w, L.post_norm_w = ptr(t["in_norm"]), ptr(t["post_norm"])
    L.q_norm_w, L.k_norm_w = ptr(t["q_norm"]), ptr(t["k_norm"])
    L.w_qkv, L.w_o, L.w_gu, L.w_down = ptr(t["w_qkv"]), ptr(t["w_o"]), ptr(t["w_gu"]), ptr(t["w_down"])
    if wtype == HR_FP8_E4M3:
        L.ws_qkv, L.ws_o = ptr(wscales["qkv"]), ptr(wscales["o"])
        L.ws_gu, L.ws_down = ptr(wscales["gu"]), ptr(wscales["dn"])
        L.as_qkv, L.as_o, L.as_gu, L.as_down = (scales["qkv"], scales["o"], scales["gu"], scales["dn"])
    if wtype == HR_MXFP4:
        L.mx_o_s, L.mx_gu_s, L.mx_down_s = ptr(mx["o_s"]), ptr(mx["gu_s"]), ptr(mx["down_s"])
        L.awq_inv_o, L.awq_inv_gu = ptr(mx.get("inv_o")), ptr(mx.get("inv_gu"))
    L._tensors = (t, wscales, mx)     # raw pointers above: keep the weights alive with the struct
    return L


# ---------------------------------------------------------------------------- the C entry points
def hr_workspace_bytes(dims: HrDims, wtype: int, total_tokens: int) -> int:
    return lib().hr_workspace_bytes(ctypes.byref(dims), wtype, total_tokens)


def hr_prefill_layer(dims, layer, batch: Batch, h, kv: HrKv, ws, stream=None) -> None:
    _check(lib().hr_prefill_layer(ctypes.byref(dims), ctypes.byref(layer), ctypes.byref(batch.c), ptr(h),
                                  ctypes.byref(kv), ptr(ws), ws.numel() * ws.element_size(),
                                  stream if stream is not None else current_stream()))


def hr_prefill_stack(dims, layers: list, batch: Batch, ids, embed, vocab, x_embeds, kvs: list, final_norm_w,
                     head_w, n_codebooks, cb_vocab, h_out, logits_out, ws, stream=None) -> None:
    L = (HrLayer * len(layers))(*layers)
    K = (HrKv * len(kvs))(*kvs)
    _check(lib().hr_prefill_stack(ctypes.byref(dims), L, ctypes.byref(batch.c), ptr(ids), ptr(embed), vocab,
                                  ptr(x_embeds), K, ptr(final_norm_w), ptr(head_w), n_codebooks, cb_vocab,
                                  ptr(h_out), ptr(logits_out), ptr(ws), ws.numel() * ws.element_size(),
                                  stream if stream is not None else current_stream()))


def hr_decode_workspace_bytes(dims: HrDims, wtype: int, B: int) -> int:
    return lib().hr_decode_workspace_bytes(ctypes.byref(dims), wtype, B)


def hr_decode_step(dims, layers: list, batch: Batch, x_embeds, kvs: list, final_norm_w, head_w, n_codebooks,
                   cb_vocab, bos_id, eoc_id, logits_out, frame, eoc_seen, done, codes, aligned, max_frames,
                   cb_embed, emb_out, ws, stream=None) -> None:
    L = (HrLayer * len(layers))(*layers)
    K = (HrKv * len(kvs))(*kvs)
    _check(lib().hr_decode_step(ctypes.byref(dims), L, ctypes.byref(batch.c), ptr(x_embeds), K, ptr(final_norm_w),
                                ptr(head_w), n_codebooks, cb_vocab, bos_id, eoc_id, ptr(logits_out), ptr(frame),
                                ptr(eoc_seen), ptr(done), ptr(codes), ptr(aligned), max_frames, ptr(cb_embed),
                                ptr(emb_out), ptr(ws), ws.numel() * ws.element_size(),
                                stream if stream is not None else current_stream()))


def hr_decode_noalloc_scratch_bytes() -> int:
    return lib().hr_decode_noalloc_scratch_bytes()


def hr_decode_step_noalloc(dims, layers: list, batch: Batch, x_embeds, kvs: list, final_norm_w, head_w,
                           n_codebooks, cb_vocab, bos_id, eoc_id, logits_out, frame, eoc_seen, done, codes, aligned,
                           max_frames, cb_embed, emb_out, stream=None) -> None:
    L = (HrLayer * len(layers))(*layers)
    K = (HrKv * len(kvs))(*kvs)
    _check(lib().hr_decode_step_noalloc(ctypes.byref(dims), L, ctypes.byref(batch.c), ptr(x_embeds), K,
                                        ptr(final_norm_w), ptr(head_w), n_codebooks, cb_vocab, bos_id, eoc_id,
                                        ptr(logits_out), ptr(frame), ptr(eoc_seen), ptr(done), ptr(codes), ptr(aligned),
                                        max_frames, ptr(cb_embed), ptr(emb_out),
                                        stream if stream is not None else current_stream()))


def hr_codebook_step(B, K, V, bos_id, eoc_id, logits, frame, eoc_seen, done, codes, aligned, max_frames,
                     cb_embed, D, emb_out, stream=None) -> None:
    import torch
    f32 = 1 if logits.dtype == torch.float32 else 0
    _check(lib().hr_codebook_step(B, K, V, bos_id, eoc_id, f32, ptr(logits), ptr(frame), ptr(eoc_seen),
                                  ptr(done), ptr(codes), ptr(aligned), max_frames, ptr(cb_embed), D,
                                  ptr(emb_out), stream if stream is not None else current_stream()))


def make_policy(temperature=None, top_k=None, top_p=None, seed=None, eoc_cascade=False, repeat_limit=0,
                end_frame=None, last_codes=None, repeat_run=None) -> HrStepPolicy:
    """hr_step_policy over device tensors (kept alive on the returned struct)."""
    pol = HrStepPolicy(ptr(temperature), ptr(top_k), ptr(top_p), ptr(seed), 1 if eoc_cascade else 0,
                       int(repeat_limit), ptr(end_frame), ptr(last_codes), ptr(repeat_run))
    pol._tensors = (temperature, top_k, top_p, seed, end_frame, last_codes, repeat_run)
    return pol


def hr_codebook_step_policy(B, K, V, bos_id, eoc_id, logits, frame, eoc_seen, done, codes, aligned, max_frames,
                            cb_embed, D, emb_out, policy=None, stream=None) -> None:
    import torch
    f32 = 1 if logits.dtype == torch.float32 else 0
    _check(lib().hr_codebook_step_policy(B, K, V, bos_id, eoc_id, f32, ptr(logits), ptr(frame), ptr(eoc_seen),
                                         ptr(done), ptr(codes), ptr(aligned), max_frames, ptr(cb_embed), D,
                                         ptr(emb_out), ctypes.byref(policy) if policy is not None else None,
                                         stream if stream is not None else current_stream()))


def hr_embed_rmsnorm(ids, embed, vocab, x_embeds, T, D, norm_w, eps, h_out, x_out, x_type=HR_F16,
                     x_scale=1.0, stream=None) -> None:
    _check(lib().hr_embed_rmsnorm(ptr(ids), ptr(embed), vocab, ptr(x_embeds), T, D, ptr(norm_w), eps,
                                  ptr(h_out), ptr(x_out), x_type, x_scale,
                                  stream if stream is not None else current_stream()))


def hr_rmsnorm(h, T, D, norm_w, eps, x_out, x_type=HR_F16, x_scale=1.0, stream=None) -> None:
    _check(lib().hr_rmsnorm(ptr(h), T, D, ptr(norm_w), eps, ptr(x_out), x_type, x_scale,
                            stream if stream is not None else current_stream()))


def hr_linear_workspace_bytes(wtype, M, N, K, epi) -> int:
    return lib().hr_linear_workspace_bytes(wtype, M, N, K, epi)


def hr_pack_weight(w, N, K, gate_up, out, stream=None) -> None:
    """bf16 w [N, K] -> ``out`` (N * K * 2 bytes) for HR_F16_PACKED layers."""
    _check(lib().hr_pack_weight(ptr(w), N, K, int(gate_up), ptr(out),
                                stream if stream is not None else current_stream()))


def pack_layer_weights(t: dict, shapes: dict) -> dict:
    """Copy of layer dict ``t`` with w_qkv / w_o / w_gu / w_down replaced by
    their packed forms; ``shapes[name] = (N, K)``."""
    import torch
    out = dict(t)
    for name in ("w_qkv", "w_o", "w_gu", "w_down"):
        N, K = shapes[name]
        p = torch.empty((N, K), dtype=torch.float16, device=t[name].device)
        hr_pack_weight(t[name], N, K, name == "w_gu", p)
        out[name] = p
    return out


def hr_linear(x, w, w_scale, x_scale, wtype, M, N, K, epi, out, out_scale=0.0, ws=None, stream=None) -> None:
    """``ws``: device scratch of hr_linear_workspace_bytes(...) bytes (a torch
    tensor) when that is non-zero (the split-K partials of HR_EPI_RESIDUAL)."""
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hr_linear(ptr(x), ptr(w), ptr(w_scale), x_scale, wtype, M, N, K, epi, ptr(out), out_scale,
                           ptr(ws), nbytes, stream if stream is not None else current_stream()))


def hr_residual_rmsnorm(h, partials, n_partials, T, D, norm_w, eps, x_out, x_type=HR_F16, x_scale=1.0,
                        stream=None) -> None:
    _check(lib().hr_residual_rmsnorm(ptr(h), ptr(partials), n_partials, T, D, ptr(norm_w), eps, ptr(x_out), x_type,
                                     x_scale, stream if stream is not None else current_stream()))


def hr_qknorm_rope_kv(dims, batch: Batch, qkv, q_norm_w, k_norm_w, q_out, kv: HrKv, stream=None) -> None:
    _check(lib().hr_qknorm_rope_kv(ctypes.byref(dims), ctypes.byref(batch.c), ptr(qkv), ptr(q_norm_w),
                                   ptr(k_norm_w), ptr(q_out), ctypes.byref(kv),
                                   stream if stream is not None else current_stream()))


def hr_attention(dims, batch: Batch, q, kv: HrKv, out, out_type=HR_F16, out_scale=1.0, stream=None) -> None:
    _check(lib().hr_attention(ctypes.byref(dims), ctypes.byref(batch.c), ptr(q), ctypes.byref(kv), ptr(out),
                              out_type, out_scale, stream if stream is not None else current_stream()))


def hr_attention_f16(dims, batch: Batch, q, k16, v16, Tp, out, out_type=HR_F16, out_scale=1.0, stream=None) -> None:
    _check(lib().hr_attention_f16(ctypes.byref(dims), ctypes.byref(batch.c), ptr(q), ptr(k16), ptr(v16), Tp,
                                  ptr(out), out_type, out_scale,
                                  stream if stream is not None else current_stream()))


def hr_qknorm_rope_attention(dims, batch: Batch, qkv, q_norm_w, k_norm_w, kv: HrKv, out, out_type=HR_F16,
                             out_scale=1.0, stream=None) -> None:
    _check(lib().hr_qknorm_rope_attention(ctypes.byref(dims), ctypes.byref(batch.c), ptr(qkv), ptr(q_norm_w),
                                          ptr(k_norm_w), ctypes.byref(kv), ptr(out), out_type, out_scale,
                                          stream if stream is not None else current_stream()))


def hr_attention_chunked_workspace_bytes(dims, total_tokens: int, n_slots: int) -> int:
    return lib().hr_attention_chunked_workspace_bytes(ctypes.byref(dims), total_tokens, n_slots)


def hr_attention_chunked(dims, batch: Batch, q, kv: HrKv, out, chunk_tiles: int, n_slots: int, ws,
                         out_type=HR_F16, out_scale=1.0, stream=None) -> None:
    _check(lib().hr_attention_chunked(ctypes.byref(dims), ctypes.byref(batch.c), ptr(q), ctypes.byref(kv), ptr(out),
                                      out_type, out_scale, chunk_tiles, n_slots, ptr(ws),
                                      ws.numel() * ws.element_size(),
                                      stream if stream is not None else current_stream()))


def hr_head_workspace_bytes(n_seq: int, D: int) -> int:
    return lib().hr_head_workspace_bytes(n_seq, D)


def hr_head_logits(h, batch: Batch, D, final_norm_w, eps, head_w, n_codebooks, cb_vocab, logits_out, ws,
                   stream=None) -> None:
    _check(lib().hr_head_logits(ptr(h), ctypes.byref(batch.c), D, ptr(final_norm_w), eps, ptr(head_w),
                                n_codebooks, cb_vocab, ptr(logits_out), ptr(ws), ws.numel() * ws.element_size(),
                                stream if stream is not None else current_stream()))


def hr_quantize_weight_e4m3(w, N, K, w8, scale, stream=None) -> None:
    _check(lib().hr_quantize_weight_e4m3(ptr(w), N, K, ptr(w8), ptr(scale),
                                         stream if stream is not None else current_stream()))


def mx_scale_bytes(rows: int, K: int) -> int:
    """Bytes of an MXFP4 scale array of ``rows`` rows (ld = rows) over K."""
    return (K // 128) * rows * 4


def hr_quantize_mxfp4(x, M, K, codes, scales, ld_scales, col_scale=None, row_scale=None, stream=None) -> None:
    import torch
    fmt = {torch.bfloat16: MX_SRC_BF16, torch.float32: MX_SRC_F32, torch.float16: MX_SRC_F16}[x.dtype]
    _check(lib().hr_quantize_mxfp4(ptr(x), fmt, M, K, ptr(col_scale), ptr(row_scale), ptr(codes), ptr(scales),
                                   ld_scales, stream if stream is not None else current_stream()))


def hr_rmsnorm_mxfp4(h, T, D, norm_w, eps, codes, scales, ld_scales, col_scale=None, stream=None) -> None:
    _check(lib().hr_rmsnorm_mxfp4(ptr(h), T, D, ptr(norm_w), eps, ptr(col_scale), ptr(codes), ptr(scales),
                                  ld_scales, stream if stream is not None else current_stream()))


def hr_linear_mxfp4(x, x_scales, ld_x_scales, w, w_scales, M, N, K, epi, out, out_scales=None, ld_out_scales=0,
                    ws=None, stream=None) -> None:
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hr_linear_mxfp4(ptr(x), ptr(x_scales), ld_x_scales, ptr(w), ptr(w_scales), M, N, K, epi,
                                 ptr(out), ptr(out_scales), ld_out_scales, ptr(ws), nbytes,
                                 stream if stream is not None else current_stream()))


def linear_ws(wtype, M, N, K, epi):
    """A device workspace for hr_linear / hr_linear_mxfp4 (None when none is needed)."""
    import torch
    n = hr_linear_workspace_bytes(wtype, M, N, K, epi)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
