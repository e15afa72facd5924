"""The C ABI on the CPU: libhr.so loads, exports every function include/*.h
declares, and refuses bad calls on the host before any launch.

Every call here carries exactly one planted error, so validation returns before
a kernel could run; the device pointers are fake (aligned, never dereferenced).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import codebook_decode_amd.hr as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000           # 16-byte aligned, never dereferenced
MISALIGNED = 0x100008


def declared_functions():
    names = set()
    for hdr in ("hr.h", "hr_ops.h"):
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(hr_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = H.lib()
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert {"hr_prefill_layer", "hr_prefill_stack", "hr_codebook_step"} <= set(names)


def dims(causal=True, **kw):
    d = dict(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728, n_layers=2,
             rope_theta=1e6, rms_eps=1e-6, causal=causal)
    d.update(kw)
    return H.make_dims(**d)


def layer(**kw):
    L = H.HrLayer()
    L.wtype = H.HR_BF16
    for f in ("in_norm_w", "post_norm_w", "q_norm_w", "k_norm_w", "w_qkv", "w_o", "w_gu", "w_down"):
        setattr(L, f, FAKE)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def batch(lens, starts=None, slots=None, used=None, max_seqlen=None):
    n = len(lens)
    return H.Batch(np.concatenate([[0], np.cumsum(lens)]), starts or [0] * n, slots or list(range(n)), used,
                   max_seqlen, device="cpu")


def kv(capacity=2048, n_slots=4, **kw):
    k = H.HrKv(FAKE, FAKE, capacity, n_slots)
    for a, v in kw.items():
        setattr(k, a, v)
    return k


def call_layer(d, L, b, kvv, ws_bytes=1 << 40, h=FAKE, ws=FAKE):
    lib = H.lib()
    return lib.hr_prefill_layer(ctypes.byref(d), ctypes.byref(L), ctypes.byref(b.c), h, ctypes.byref(kvv), ws,
                                ws_bytes, None)


@pytest.mark.parametrize("case,status", [
    ("head_dim", H.HR_EUNSUPPORTED), ("group", H.HR_EUNSUPPORTED), ("hidden", H.HR_EUNSUPPORTED),
    ("null_weight", H.HR_EINVAL), ("misaligned_weight", H.HR_EALIGN), ("capacity", H.HR_ECAPACITY),
    ("slot", H.HR_ECAPACITY), ("max_seqlen", H.HR_EBOUND), ("used_gt_len", H.HR_EBOUND),
    ("used_missing", H.HR_EINVAL), ("cu_not_monotone", H.HR_EINVAL), ("workspace", H.HR_EWORKSPACE),
    ("misaligned_h", H.HR_EALIGN), ("fp8_scale", H.HR_EINVAL), ("noncausal_start", H.HR_EUNSUPPORTED),
    ("weight_4gb", H.HR_EUNSUPPORTED), ("activation_4gb", H.HR_EUNSUPPORTED),
    ("fp8_k64", H.HR_EUNSUPPORTED),
])
def test_prefill_layer_validation(case, status):
    d, L, b, k = dims(), layer(), batch([13]), kv()
    ws_bytes, h = 1 << 40, FAKE
    if case == "head_dim":
        d = dims(head_dim=96)
    elif case == "group":
        d = dims(n_kv_heads=4)                      # 8 query heads per kv head
    elif case == "hidden":
        d = dims(hidden=2500)
    elif case == "null_weight":
        L = layer(w_gu=None)
    elif case == "misaligned_weight":
        L = layer(w_o=MISALIGNED)
    elif case == "capacity":
        b = batch([13], starts=[2040])
    elif case == "slot":
        b = batch([13, 4], slots=[0, 4])
    elif case == "max_seqlen":
        b = batch([13, 20], max_seqlen=16)
    elif case == "used_gt_len":
        d, b = dims(causal=False), batch([13], used=[14])
    elif case == "used_missing":
        d = dims(causal=False)
    elif case == "cu_not_monotone":
        b = H.Batch(np.array([0, 5, 3]), [0, 0], [0, 1], device="cpu")
    elif case == "workspace":
        ws_bytes = H.hr_workspace_bytes(d, H.HR_BF16, 13) - 1
    elif case == "misaligned_h":
        h = MISALIGNED
    elif case == "fp8_scale":
        L = layer(wtype=H.HR_FP8_E4M3, ws_qkv=FAKE, ws_o=FAKE, ws_gu=FAKE, ws_down=FAKE,
                  as_qkv=1.0, as_o=0.0, as_gu=1.0, as_down=1.0)
    elif case == "fp8_k64":                          # e4m3 K steps of 128 values: F = 9664 is not one
        d = dims(ffn=9664)
        L = layer(wtype=H.HR_FP8_E4M3, ws_qkv=FAKE, ws_o=FAKE, ws_gu=FAKE, ws_down=FAKE,
                  as_qkv=1.0, as_o=1.0, as_gu=1.0, as_down=1.0)
    elif case == "noncausal_start":
        d, b = dims(causal=False), batch([13], starts=[4], used=[13])
    elif case == "weight_4gb":                       # 2F x D bf16 gate/up >= 4 GB
        d = dims(hidden=8192, n_q_heads=64, n_kv_heads=16, ffn=131072)
    elif case == "activation_4gb":                   # T x F bf16 >= 4 GB
        b, k = batch([230000], max_seqlen=230000), kv(capacity=1 << 20)
    st = call_layer(d, L, b, k, ws_bytes, h)
    assert st == status, (case, st, H.hr_last_error())
    assert H.hr_last_error()
    if case.endswith("4gb"):
        assert "4 GB" in H.hr_last_error(), H.hr_last_error()


def test_empty_batch_is_a_no_op():
    assert call_layer(dims(), layer(), batch([0]), kv()) == H.HR_OK


def test_workspace_bytes_grow_with_tokens():
    d = dims()
    a, b = H.hr_workspace_bytes(d, H.HR_BF16, 13), H.hr_workspace_bytes(d, H.HR_BF16, 512)
    assert 0 < a < b
    per_tok = (2560 * 2 + 6144 * 2 + 4096 * 2 * 2 + 9728 * 2)
    assert b >= 512 * per_tok


def test_stack_validation():
    lib = H.lib()
    d = dims()
    Ls = (H.HrLayer * 2)(layer(), layer(wtype=H.HR_FP8_E4M3, ws_qkv=FAKE, ws_o=FAKE, ws_gu=FAKE, ws_down=FAKE,
                                        as_qkv=1.0, as_o=1.0, as_gu=1.0, as_down=1.0))
    Ks = (H.HrKv * 2)(kv(), kv())
    b = batch([13])
    st = lib.hr_prefill_stack(ctypes.byref(d), Ls, ctypes.byref(b.c), FAKE, FAKE, 151936, None, Ks, FAKE, None,
                              8, 1026, FAKE, None, FAKE, 1 << 40, None)
    assert st == H.HR_EINVAL and "wtype" in H.hr_last_error()
    Ls2 = (H.HrLayer * 2)(layer(), layer())
    st = lib.hr_prefill_stack(ctypes.byref(d), Ls2, ctypes.byref(b.c), FAKE, FAKE, 151936, None, Ks, FAKE, FAKE,
                              8, 1026, FAKE, None, FAKE, 1 << 40, None)
    assert st == H.HR_EINVAL and "head_w" in H.hr_last_error()
    b0 = batch([3, 0, 2])
    st = lib.hr_prefill_stack(ctypes.byref(d), Ls2, ctypes.byref(b0.c), FAKE, FAKE, 151936, None, Ks, FAKE, FAKE,
                              8, 1026, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == H.HR_EINVAL and "empty" in H.hr_last_error()


@pytest.mark.parametrize("B,K,V,bos,eoc,D,status", [
    (4, 8, 1026, 1024, 1024, 2560, H.HR_EINVAL),     # bos == eoc
    (4, 8, 1026, 1024, 1026, 2560, H.HR_EINVAL),     # eoc out of range
    (4, 8, 1026, -1, 1025, 2560, H.HR_EINVAL),
    (4, 8, 1026, 1024, 1025, 2561, H.HR_EINVAL),     # D not a multiple of 8
    (4, 0, 1026, 1024, 1025, 2560, H.HR_EINVAL),
    (4, 2000, 1026, 1024, 1025, 2560, H.HR_EUNSUPPORTED),
])
def test_codebook_validation(B, K, V, bos, eoc, D, status):
    lib = H.lib()
    st = lib.hr_codebook_step(B, K, V, bos, eoc, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, D, FAKE, None)
    assert st == status, H.hr_last_error()


def test_codebook_misaligned_embedding_refused():
    lib = H.lib()
    st = lib.hr_codebook_step(4, 8, 1026, 1024, 1025, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, MISALIGNED, 2560,
                              FAKE, None)
    assert st == H.HR_EALIGN


def test_linear_validation():
    lib = H.lib()
    # an operand of 4 GB or more (32-bit byte offsets in the tiled GEMM)
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 65536, 64, 32768, 0, FAKE, 0.0, None, 0, None) == \
        H.HR_EUNSUPPORTED
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 4, 16, 48, 0, FAKE, 0.0, None, 0, None) == H.HR_EUNSUPPORTED
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 4, 24, 64, 0, FAKE, 0.0, None, 0, None) == H.HR_EUNSUPPORTED
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_FP8_E4M3, 4, 16, 128, 0, FAKE, 0.0, None, 0, None) == H.HR_EINVAL
    assert lib.hr_linear(FAKE, FAKE, FAKE, 1.0, H.HR_FP8_E4M3, 4, 32, 128, 2, FAKE, 0.0, None, 0, None) == H.HR_EINVAL
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 4, 16, 64, 7, FAKE, 0.0, None, 0, None) == H.HR_EINVAL
    # a residual projection that splits K needs the partial workspace
    assert H.hr_linear_workspace_bytes(H.HR_BF16, 13, 2560, 9728, H.HR_EPI_RESIDUAL) > 0
    assert H.hr_linear_workspace_bytes(H.HR_BF16, 13, 2560, 9728, H.HR_EPI_F32) == 0
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 13, 2560, 9728, 1, FAKE, 0.0, None, 0, None) == \
        H.HR_EWORKSPACE
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_BF16, 13, 2560, 9728, 1, FAKE, 0.0, FAKE, 100, None) == \
        H.HR_EWORKSPACE


def test_pack_weight_validation():
    lib = H.lib()
    f = lib.hr_pack_weight
    assert f(FAKE, 64, 48, 0, FAKE + (1 << 20), None) == H.HR_EINVAL          # K % 32
    assert f(FAKE, 0, 64, 0, FAKE + (1 << 20), None) == H.HR_EINVAL
    assert f(FAKE, 96, 64, 1, FAKE + (1 << 20), None) == H.HR_EUNSUPPORTED    # gate/up: N % 64
    assert f(FAKE, 64, 64, 2, FAKE + (1 << 20), None) == H.HR_EINVAL          # gate_up flag 0 / 1
    assert f(None, 64, 64, 0, FAKE, None) == H.HR_EINVAL
    assert f(FAKE, 64, 64, 0, MISALIGNED, None) == H.HR_EALIGN
    assert f(FAKE, 64, 64, 0, FAKE + 4096, None) == H.HR_EINVAL               # out overlaps w
    assert f(FAKE, 65536, 32768, 0, FAKE + (1 << 40), None) == H.HR_EUNSUPPORTED   # >= 2 GB
    # a packed layer and hr_linear accept the format, with the gate/up rule
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, H.HR_F16_PACKED, 4, 96, 64, 2, FAKE, 0.0, None, 0, None) == \
        H.HR_EUNSUPPORTED
    assert lib.hr_linear(FAKE, FAKE, None, 1.0, 5, 4, 64, 64, 0, FAKE, 0.0, None, 0, None) == H.HR_EINVAL


def test_residual_rmsnorm_validation():
    lib = H.lib()
    f = lib.hr_residual_rmsnorm
    assert f(FAKE, FAKE, -1, 4, 256, FAKE, 1e-6, FAKE, H.HR_F16, 1.0, None) == H.HR_EINVAL
    assert f(FAKE, None, 2, 4, 256, FAKE, 1e-6, FAKE, H.HR_F16, 1.0, None) == H.HR_EINVAL      # partials missing
    assert f(FAKE, FAKE, 2, 4, 250, FAKE, 1e-6, FAKE, H.HR_F16, 1.0, None) == H.HR_EINVAL      # D % 8
    assert f(FAKE, FAKE, 2, 4, 256, FAKE, 1e-6, FAKE, H.HR_BF16, 1.0, None) == H.HR_EINVAL     # x fp16 or e4m3
    assert f(FAKE, FAKE, 2, 4, 256, FAKE, 1e-6, FAKE, H.HR_FP8_E4M3, 0.0, None) == H.HR_EINVAL
    assert f(FAKE, FAKE, 2, 4, 256, None, 1e-6, FAKE, H.HR_F16, 1.0, None) == H.HR_EINVAL      # norm weight
    assert f(MISALIGNED, FAKE, 2, 4, 256, FAKE, 1e-6, FAKE, H.HR_F16, 1.0, None) == H.HR_EALIGN


def test_codebook_misaligned_logits_refused():
    lib = H.lib()
    st = lib.hr_codebook_step(4, 8, 1026, 1024, 1025, 0, MISALIGNED, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 2560,
                              FAKE, None)
    assert st == H.HR_EALIGN


@pytest.mark.parametrize("case,status", [
    ({"V": 2049}, H.HR_EUNSUPPORTED),
    ({"temperature": FAKE}, H.HR_EINVAL),                        # temperature without seed
    ({"temperature": FAKE, "seed": FAKE + 4}, H.HR_EALIGN),
    ({"repeat_limit": 1, "end_frame": FAKE, "last_codes": FAKE, "repeat_run": FAKE}, H.HR_EINVAL),
    ({"repeat_limit": -2, "end_frame": FAKE, "last_codes": FAKE, "repeat_run": FAKE}, H.HR_EINVAL),
    ({"eoc_cascade": 1}, H.HR_EINVAL),                           # no end_frame
    ({"repeat_limit": 4, "end_frame": FAKE}, H.HR_EINVAL),       # no guard state
    ({"repeat_limit": 4, "end_frame": FAKE, "last_codes": FAKE}, H.HR_EINVAL),
    ({"bos": 1026}, H.HR_EINVAL),                                # the plain step's checks still apply
])
def test_codebook_policy_validation(case, status):
    lib = H.lib()
    c = dict(case)
    V = c.pop("V", 1026)
    bos = c.pop("bos", V - 2)
    pol = H.HrStepPolicy(c.get("temperature"), None, None, c.get("seed"), c.get("eoc_cascade", 0),
                         c.get("repeat_limit", 0), c.get("end_frame"), c.get("last_codes"), c.get("repeat_run"))
    st = lib.hr_codebook_step_policy(4, 8, V, bos, V - 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 2560,
                                     FAKE, ctypes.byref(pol), None)
    assert st == status, (st, H.hr_last_error())


def test_mxfp4_validation():
    lib = H.lib()
    # the bf16 / e4m3 entries refuse the MXFP4 type
    assert lib.hr_rmsnorm(FAKE, 4, 256, FAKE, 1e-6, FAKE, H.HR_MXFP4, 1.0, None) == H.HR_EINVAL
    # norm outputs are fp16 (the bf16-weight band) or e4m3
    assert lib.hr_rmsnorm(FAKE, 4, 256, FAKE, 1e-6, FAKE, H.HR_BF16, 1.0, None) == H.HR_EINVAL
    # K not a multiple of 128; ld below M
    assert lib.hr_quantize_mxfp4(FAKE, 0, 4, 96, None, None, FAKE, FAKE, 4, None) == H.HR_EINVAL
    assert lib.hr_quantize_mxfp4(FAKE, 0, 8, 128, None, None, FAKE, FAKE, 4, None) == H.HR_EINVAL
    assert lib.hr_rmsnorm_mxfp4(FAKE, 4, 200, FAKE, 1e-6, None, FAKE, FAKE, 4, None) == H.HR_EINVAL
    lin = lib.hr_linear_mxfp4
    # x scales must cover the 256-row tiles; N multiple of 256; bf16 epilogue refused
    assert lin(FAKE, FAKE, 100, FAKE, FAKE, 100, 256, 256, H.HR_EPI_RESIDUAL, FAKE, None, 0, None, 0, None) == H.HR_EINVAL
    assert lin(FAKE, FAKE, 256, FAKE, FAKE, 100, 384, 256, H.HR_EPI_RESIDUAL, FAKE, None, 0, None, 0, None) == \
        H.HR_EUNSUPPORTED
    assert lin(FAKE, FAKE, 256, FAKE, FAKE, 100, 256, 256, H.HR_EPI_F32, FAKE, None, 0, None, 0, None) == H.HR_EINVAL
    # the quantiser's source format is 0 (bf16), 1 (fp32) or 2 (fp16)
    assert lib.hr_quantize_mxfp4(FAKE, 3, 4, 128, None, None, FAKE, FAKE, 4, None) == H.HR_EINVAL
    assert lin(FAKE, FAKE, 256, FAKE, FAKE, 100, 512, 256, H.HR_EPI_SWIGLU, FAKE, None, 0, None, 0, None) == H.HR_EINVAL
    assert lin(FAKE, FAKE, 256, FAKE, FAKE, 100, 512, 256, H.HR_EPI_SWIGLU, FAKE, FAKE, 128, None, 0, None) == H.HR_EINVAL
    assert lin(FAKE, FAKE, 256, FAKE, FAKE, 100, 512, 200, H.HR_EPI_SWIGLU, FAKE, FAKE, 256, None, 0, None) == H.HR_EINVAL
    assert lin(FAKE + 4, FAKE, 256, FAKE, FAKE, 100, 512, 256, H.HR_EPI_SWIGLU, FAKE, FAKE, 256, None, 0, None) == \
        H.HR_EALIGN


@pytest.mark.parametrize("ct,slots,ws,ws_bytes,status", [
    (0, 4, FAKE, 1 << 40, H.HR_EINVAL),           # chunk_tiles < 1
    (2, 0, FAKE, 1 << 40, H.HR_EINVAL),           # no slot
    (2, 65, FAKE, 1 << 40, H.HR_EINVAL),          # too many slots
    (2, 4, FAKE, 1000, H.HR_EWORKSPACE),
    (2, 4, None, 1 << 40, H.HR_EWORKSPACE),
    (2, 4, FAKE + 16, 1 << 40, H.HR_EALIGN),
])
def test_attention_chunked_validation(ct, slots, ws, ws_bytes, status):
    lib = H.lib()
    d, b, k = dims(), batch([300]), kv()
    st = lib.hr_attention_chunked(ctypes.byref(d), ctypes.byref(b.c), FAKE, ctypes.byref(k), FAKE, H.HR_F16, 1.0,
                                  ct, slots, ws, ws_bytes, None)
    assert st == status, (st, H.hr_last_error())
    assert H.hr_attention_chunked_workspace_bytes(d, 300, 4) >= 4 * 300 * 32 * (128 * 4 + 8)


@pytest.mark.parametrize("case,status", [
    ("ok", H.HR_OK),                            # zero rows: validated, nothing launched
    ("continuation", H.HR_EUNSUPPORTED),        # a sequence past position 0: keys in the cache
    ("start_row", H.HR_EUNSUPPORTED),           # a sequence starting at batch row 13 (not a multiple of 8)
    ("tp_small", H.HR_EINVAL),                  # Tp below T rounded up to 32
    ("tp_ragged", H.HR_EINVAL),                 # Tp not a multiple of 32
    ("misaligned", H.HR_EALIGN),
    ("no_copy", H.HR_EINVAL),
    ("fp8_scale", H.HR_EINVAL),
])
def test_attention_f16_validation(case, status):
    lib = H.lib()
    d = dims()
    lens = [0] if case == "ok" else ([13, 5] if case == "start_row" else [16, 5])
    b = batch(lens, starts=[0, 7] if case == "continuation" else None)
    T = sum(lens)
    Tp = {"tp_small": 0 if T <= 32 else 32, "tp_ragged": 48}.get(case, (T + 31) // 32 * 32 or 32)
    k16 = None if case == "no_copy" else (FAKE + 8 if case == "misaligned" else FAKE)
    out_type = H.HR_FP8_E4M3 if case == "fp8_scale" else H.HR_F16
    scale = 0.0 if case == "fp8_scale" else 1.0
    st = lib.hr_attention_f16(ctypes.byref(d), ctypes.byref(b.c), FAKE, k16, FAKE, Tp, FAKE, out_type, scale, None)
    assert st == status, (st, H.hr_last_error())


@pytest.mark.parametrize("case,status", [
    ("continuation", H.HR_EUNSUPPORTED),        # a sequence past position 0
    ("long", H.HR_EUNSUPPORTED),                # 33 rows
    ("out_type", H.HR_EINVAL),
    ("out_bf16", H.HR_EINVAL),                  # activations of the bf16-weight band are fp16
    ("fp8_scale", H.HR_EINVAL),
    ("no_out", H.HR_EINVAL),
])
def test_qknorm_rope_attention_validation(case, status):
    lib = H.lib()
    d, k = dims(), kv()
    b = batch([13, 33] if case == "long" else [13, 5], starts=[0, 7] if case == "continuation" else None)
    out_type = {"out_type": H.HR_MXFP4, "fp8_scale": H.HR_FP8_E4M3, "out_bf16": H.HR_BF16}.get(case, H.HR_F16)
    scale = 0.0 if case == "fp8_scale" else 1.0
    out = None if case == "no_out" else FAKE
    st = lib.hr_qknorm_rope_attention(ctypes.byref(d), ctypes.byref(b.c), FAKE, FAKE, FAKE, ctypes.byref(k), out,
                                      out_type, scale, None)
    assert st == status, (st, H.hr_last_error())


@pytest.mark.parametrize("case,status", [
    ("noncausal", H.HR_EUNSUPPORTED), ("two_rows", H.HR_EINVAL), ("no_head", H.HR_EINVAL),
    ("bos_eq_eoc", H.HR_EINVAL), ("workspace", H.HR_EWORKSPACE), ("misaligned_emb", H.HR_EALIGN),
    ("capacity", H.HR_ECAPACITY), ("wtype_mix", H.HR_EINVAL),
])
def test_decode_step_validation(case, status):
    lib = H.lib()
    d = dims()
    Ls = (H.HrLayer * 2)(layer(), layer())
    Ks = (H.HrKv * 2)(kv(), kv())
    b = batch([1, 1, 1], starts=[10, 200, 5])
    head, emb, bos, ws_bytes = FAKE, FAKE, 1024, 1 << 40
    if case == "noncausal":
        d, b = dims(causal=False), batch([1, 1, 1], used=[1, 1, 1])
    elif case == "two_rows":
        b = batch([1, 2, 1], starts=[10, 200, 5])
    elif case == "no_head":
        head = None
    elif case == "bos_eq_eoc":
        bos = 1025
    elif case == "workspace":
        ws_bytes = H.hr_decode_workspace_bytes(d, H.HR_BF16, 3) - 1
    elif case == "misaligned_emb":
        emb = MISALIGNED
    elif case == "capacity":
        b = batch([1, 1, 1], starts=[2048, 200, 5])
    elif case == "wtype_mix":
        Ls = (H.HrLayer * 2)(layer(), layer(wtype=H.HR_FP8_E4M3, ws_qkv=FAKE, ws_o=FAKE, ws_gu=FAKE,
                                           ws_down=FAKE, as_qkv=1.0, as_o=1.0, as_gu=1.0, as_down=1.0))
    st = lib.hr_decode_step(ctypes.byref(d), Ls, ctypes.byref(b.c), FAKE, Ks, FAKE, head, 8, 1026, bos, 1025, FAKE,
                            FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, emb, FAKE, ws_bytes, None)
    assert st == status, (case, st, H.hr_last_error())


def test_decode_workspace_holds_the_prefill_workspace():
    d = dims()
    assert H.hr_decode_workspace_bytes(d, H.HR_BF16, 64) >= H.hr_workspace_bytes(d, H.HR_BF16, 64) + 64 * 2560 * 4


def test_decode_noalloc_validation():
    """The allocation-free decode step runs hr_decode_step's checks, and refuses
    a batch whose scratch exceeds its fixed array before touching the device."""
    lib = H.lib()
    assert H.hr_decode_noalloc_scratch_bytes() == 32 << 20
    d = dims()
    Ls = (H.HrLayer * 2)(layer(), layer())
    Ks = (H.HrKv * 2)(kv(), kv())
    call = lambda dd, b, bos=1024: lib.hr_decode_step_noalloc(
        ctypes.byref(dd), Ls, ctypes.byref(b.c), FAKE, Ks, FAKE, FAKE, 8, 1026, bos, 1025, FAKE, FAKE, FAKE, FAKE,
        FAKE, None, 0, FAKE, FAKE, None)
    assert call(dims(causal=False), batch([1, 1], used=[1, 1])) == H.HR_EUNSUPPORTED
    assert call(d, batch([1, 2], starts=[3, 4])) == H.HR_EINVAL
    assert call(d, batch([1, 1], starts=[3, 4]), bos=1025) == H.HR_EINVAL
    big = 300                                   # 4B-shape scratch of 300 streams > 32 MiB
    assert H.hr_decode_workspace_bytes(d, H.HR_BF16, big) > 32 << 20
    Kbig = (H.HrKv * 2)(kv(n_slots=big), kv(n_slots=big))
    bb = batch([1] * big, starts=[3] * big)          # kept alive: the struct points at its host arrays
    st = lib.hr_decode_step_noalloc(ctypes.byref(d), Ls, ctypes.byref(bb.c), FAKE,
                                    Kbig, FAKE, FAKE, 8, 1026, 1024, 1025, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE,
                                    FAKE, None)
    assert st == H.HR_EWORKSPACE, H.hr_last_error()


def test_one_hip_runtime_in_the_process():
    """libhr and torch share one HIP runtime: after the library is loaded, the
    process maps exactly one libamdhip64 (two runtimes in one process broke
    tensor and stream interop)."""
    H.lib()
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(libs) == 1, libs
