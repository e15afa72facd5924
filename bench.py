#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X: the 36-layer Qwen3-style 4B stack
(hidden 2560, 32/8 heads of 128, SwiGLU 9728), bf16, single prompt, batched
prefill + audio head (8 codebooks x 1026) + delayed-codebook step.

One step = hr_prefill_stack over a P=512 prompt (embedding, 36 layers with KV
writes, final norm, head logits of the last row) + hr_codebook_step on those
logits.  `value` = prompt tokens per second at P=512 (inputs resident in HBM).
The same run reports the P=13 prefill latency (ms per prompt), the dominant
kernel's roofline fraction (HIP events on the launch stream) and the CPU oracle
timed on a bounded sample.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu] [--graph]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "prefill ms/prompt at P=13, prompt tok/s at P=512; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0     # dense E2M1 (MXFP4) MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_shapes(m):
    return {"w_qkv": (m.qkv_rows, m.hidden), "w_o": (m.hidden, m.attn_width), "w_gu": (2 * m.ffn, m.hidden),
            "w_down": (m.hidden, m.ffn)}


def build_model(H, m, n_layers, keep_host=False, packed=True):
    """Seeded bf16 weights of every layer, uploaded; with `packed` also their
    hr_pack_weight form (prepared once here, outside every timed region).
    Returns the bf16 device tensors, the packed ones (or None), the layer
    structs of the timed path and (keep_host) the host bf16 bit patterns for
    the CPU oracle."""
    import torch
    import synth
    from model_util import upload_layer
    layers, dev_layers, pk_layers, host = [], [], [], []
    t0 = time.time()
    for l in range(n_layers):
        bits = synth.layer_tensors(m, l)
        dl = upload_layer(bits)
        dev_layers.append(dl)
        if packed:
            dp = H.pack_layer_weights(dl, weight_shapes(m))
            pk_layers.append(dp)
            layers.append(H.make_layer(dp, H.HR_F16_PACKED))
        else:
            layers.append(H.make_layer(dl))
        if keep_host:
            host.append(bits)
    torch.cuda.synchronize()
    log(f"weights of {n_layers} layers drawn, uploaded{' and packed' if packed else ''} in {time.time() - t0:.1f} s")
    return dev_layers, (pk_layers if packed else None), layers, host


class Stack:
    def __init__(self, H, m, P, dev_layers, layers, shared):
        import torch
        import synth
        from gpu_util import dev
        from model_util import dims_of, kv_cache, workspace
        self.H, self.m, self.P = H, m, P
        self.cap = 2048
        self.dims = dims_of(H, m, True, len(layers))
        self.layers = layers
        self.kv_t = [kv_cache(m, 1, self.cap, poison=False) for _ in layers]
        self.kv = [H.make_kv(k, v, self.cap, 1) for k, v in self.kv_t]
        self.batch = H.Batch([0, P], [0], [0])
        self.ids = dev(synth.prompt_ids(m, P))
        self.h = torch.empty((P, m.hidden), dtype=torch.float32, device="cuda")
        self.K, self.V = m.n_codebooks, m.cb_vocab
        self.logits = torch.empty((1, self.K * self.V), dtype=torch.float32, device="cuda")
        self.ws = workspace(H, self.dims, H.HR_BF16, P)
        self.sh = shared
        self.frame = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.seen = torch.zeros((1, self.K), dtype=torch.uint8, device="cuda")
        self.done = torch.zeros(1, dtype=torch.uint8, device="cuda")
        self.codes = torch.empty((1, self.K), dtype=torch.int32, device="cuda")
        self.emb = torch.empty((1, m.hidden), dtype=torch.bfloat16, device="cuda")

    def step(self):
        H, m, s = self.H, self.m, self.sh
        H.hr_prefill_stack(self.dims, self.layers, self.batch, self.ids, s["embed"], m.vocab, None, self.kv,
                           s["final"], s["head"], self.K, self.V, self.h, self.logits, self.ws)
        H.hr_codebook_step(1, self.K, self.V, m.bos_id, m.eoc_id, self.logits, self.frame, self.seen, self.done,
                           self.codes, None, 0, s["cb"], m.hidden, self.emb)


def time_steps(fn, steps, warmup, graph=False):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fn()
        torch.cuda.synchronize()
        run = g.replay
    else:
        run = fn
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_kernel_events(fn_list, reps=3):
    """Average duration of one launch, HIP events on the current stream."""
    import torch
    for fn in fn_list[:2]:
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    start.record()
    for _ in range(reps):
        for fn in fn_list:
            fn()
            n += 1
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / n


def gemm_gu_launches(H, m, P, dev_layers, wtype):
    """The gate/up + SwiGLU GEMM of the P-row prefill, one launch per layer's
    weights (in the timed path's format)."""
    import torch
    x = torch.randn((P, m.hidden), device="cuda").to(torch.float16)
    out = torch.empty((P, m.ffn), dtype=torch.float16, device="cuda")
    fns = []
    for dl in dev_layers:
        w = dl["w_gu"]
        fns.append(lambda w=w: H.hr_linear(x, w, None, 1.0, wtype, P, 2 * m.ffn, m.hidden, H.HR_EPI_SWIGLU,
                                           out))
    return fns


def gemm_traffic():
    """Bytes per launch of the gate/up GEMM from the committed FETCH_SIZE /
    WRITE_SIZE summary, if it was taken on the current GEMM source (else None)."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", "gemm_attention_p512_counters.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_t = re.search(r"traffic_bytes_per_launch: (\d+)", txt)
    m_h = re.search(r"gemm_source_sha256: ([0-9a-f]+)", txt)
    src = os.path.join(ROOT, "codebook_decode_amd", "csrc", "gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if not m_t or not m_h or m_h.group(1) != digest:
        return None
    return int(m_t.group(1))


def time_events(fn, reps, warm=2):
    """Average wall time of fn() between HIP events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / 1e3 / reps


def hbm(bytes_, sec):
    gbs = bytes_ / sec / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def layer_rotated(H, m, dev_layers, lens=(6, 13), copies=4, reps=40, wtype=None):
    """One layer at P tokens, rotating through `copies` layers' weights
    (807 MB > the 256 MB MALL, so every call streams its weights from HBM)."""
    import torch
    import synth
    from gpu_util import dev
    from model_util import dims_of, kv_cache, workspace
    dims = dims_of(H, m, True, 1)
    cap = 2048
    wtype = H.HR_BF16 if wtype is None else wtype
    layers = [H.make_layer(dl, wtype) for dl in dev_layers[:copies]]
    kvt = [kv_cache(m, 1, cap, poison=False) for _ in range(copies)]
    kvs = [H.make_kv(k, v, cap, 1) for k, v in kvt]
    weight_bytes = sum(t.numel() * t.element_size() for t in dev_layers[0].values())
    out = {"weights_mb_per_layer": round(weight_bytes / 1e6, 2), "rotated_copies": copies}
    for P in lens:
        b = H.Batch([0, P], [0], [0])
        h0 = dev(synth.bf16_bits_to_f32(synth.embed_rows(m, synth.prompt_ids(m, P))))
        h = h0.clone()
        ws = workspace(H, dims, H.HR_BF16, P)
        i = [0]

        def call():
            k = i[0] % copies
            H.hr_prefill_layer(dims, layers[k], b, h, kvs[k], ws)
            i[0] += 1
        sec = time_events(call, reps)
        out[f"p{P}"] = {"us_per_layer": round(sec * 1e6, 2), "roofline": hbm(weight_bytes, sec)}
    return out


FP8_SCALES = {"qkv": 0.010010390956675132, "o": 0.0037856422949579236, "gu": 0.010591977409446089,
              "dn": 0.021752634441032436}   # layer 0, static per-tensor: amax / 448 on the seeded 32-token prompt


def fp8_layer(H, m, dev_layer, reps=20):
    """FP8 layer of the 4B shape: 544 rows, the first 512 used, non-causal;
    e4m3 weights with per-output-channel scales packed on the device."""
    import torch
    import synth
    from gpu_util import dev
    from model_util import dims_of, fp8_pack, kv_cache, workspace
    P, rows, cap = 512, 544, 544
    w8, ws8 = fp8_pack(H, dev_layer, m)
    layer = H.make_layer(w8, H.HR_FP8_E4M3, FP8_SCALES, ws8)
    dims = dims_of(H, m, False, 1)
    kc, vc = kv_cache(m, 1, cap, poison=False)
    kv = H.make_kv(kc, vc, cap, 1)
    b = H.Batch([0, rows], [0], [0], [P])
    h0 = np.zeros((rows, m.hidden), np.float32)
    h0[:P] = synth.bf16_bits_to_f32(synth.embed_rows(m, synth.prompt_ids(m, P)))
    h = dev(h0)
    ws = workspace(H, dims, H.HR_FP8_E4M3, rows)
    sec = time_events(lambda: H.hr_prefill_layer(dims, layer, b, h, kv, ws), reps)
    e4m3_flops = 2.0 * P * m.hidden * (m.qkv_rows + 2 * m.ffn) + 2.0 * P * m.attn_width * m.hidden \
        + 2.0 * P * m.ffn * m.hidden
    attn_flops = 2.0 * 2 * m.n_q_heads * m.head_dim * P * P
    t_floor = e4m3_flops / (FP8_PEAK_TFLOPS * 1e12) + attn_flops / (BF16_PEAK_TFLOPS * 1e12)
    return {"workload": "fp8_layer_d2560_p512_pad544 (non-causal over 512 used keys)",
            "us_per_layer_wall": round(sec * 1e6, 2), "e4m3_gflop": round(e4m3_flops / 1e9, 2),
            "attention_gflop_bf16": round(attn_flops / 1e9, 2), "floor_us": round(t_floor * 1e6, 2),
            "frac_of_floor": round(t_floor / sec, 4)}


def mxfp4_layer(H, m, dev_layer, reps=20):
    """The MXFP4 band of one 4B layer at P = 512, causal: O, gate/up and down
    on E2M1 operands with E8M0 block scales (weights packed on the device; AWQ
    vectors of 1: the timing does not depend on their values), QKV and
    attention bf16."""
    import synth
    from gpu_util import dev
    from model_util import dims_of, kv_cache, mx_pack, workspace
    P, cap = 512, 512
    dl, mxd = mx_pack(H, dev_layer, m)
    layer = H.make_layer(dl, H.HR_MXFP4, mx=mxd)
    dims = dims_of(H, m, True, 1)
    kc, vc = kv_cache(m, 1, cap, poison=False)
    kv = H.make_kv(kc, vc, cap, 1)
    b = H.Batch([0, P], [0], [0])
    h = dev(synth.bf16_bits_to_f32(synth.embed_rows(m, synth.prompt_ids(m, P))))
    ws = workspace(H, dims, H.HR_MXFP4, P)
    sec = time_events(lambda: H.hr_prefill_layer(dims, layer, b, h, kv, ws), reps)
    fp4_flops = 2.0 * P * (m.attn_width * m.hidden + 2 * m.ffn * m.hidden + m.ffn * m.hidden)
    bf16_flops = 2.0 * P * m.hidden * m.qkv_rows + 2.0 * 2 * m.n_q_heads * m.head_dim * P * P / 2
    t_floor = fp4_flops / (FP4_PEAK_TFLOPS * 1e12) + bf16_flops / (BF16_PEAK_TFLOPS * 1e12)
    return {"workload": "mxfp4_layer_d2560_p512 (causal; O, gate/up, down MXFP4)",
            "us_per_layer_wall": round(sec * 1e6, 2), "fp4_gflop": round(fp4_flops / 1e9, 2),
            "bf16_gflop": round(bf16_flops / 1e9, 2), "floor_us": round(t_floor * 1e6, 2),
            "frac_of_floor": round(t_floor / sec, 4)}


def varlen_batch(H, m, layers, shared, reps=3):
    """32 prompts (lengths uniform on [6, 256], packed), 36 layers + head."""
    import torch
    import synth
    from gpu_util import dev
    from model_util import dims_of, kv_cache, workspace
    w = synth.workloads()["varlen32_stack36_d2560"]
    lens = np.array(w.prompt_lens)
    n, cap = lens.size, w.capacity
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ids = dev(np.concatenate([synth.prompt_ids(m, int(L), seq=s) for s, L in enumerate(lens)]))
    dims = dims_of(H, m, True, len(layers))
    b = H.Batch(cu, np.zeros(n), np.arange(n))
    kvt = [kv_cache(m, n, cap, poison=False) for _ in layers]
    kvs = [H.make_kv(k, v, cap, n) for k, v in kvt]
    h = torch.empty((T, m.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((n, m.n_codebooks * m.cb_vocab), dtype=torch.float32, device="cuda")
    ws = workspace(H, dims, H.HR_BF16, T)
    sec = time_events(lambda: H.hr_prefill_stack(dims, layers, b, ids, shared["embed"], m.vocab, None, kvs,
                                                 shared["final"], shared["head"], m.n_codebooks, m.cb_vocab, h,
                                                 logits, ws), reps, warm=1)
    del kvt
    return {"workload": f"varlen32_stack36_d2560: {n} prompts, T={T}, lengths {lens.min()}..{lens.max()}",
            "ms": round(sec * 1e3, 3), "tok_s": round(T / sec, 1)}


def decode_steps(H, m, dev_layers, layers, shared, B, cached, reps=5):
    """One batched decode step (hr_decode_step: the 36-layer stack over one new
    row per stream at position `cached`, the head, the codebook step), B
    streams whose caches hold `cached` rows (zeros: the values do not change
    the work).  HBM floor: the weights + head once, plus every stream's K/V
    rows of every layer."""
    import torch
    from gpu_util import dev
    from model_util import dims_of
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    cap = cached + 64
    dims = dims_of(H, m, True, len(layers))
    kvt = [(torch.zeros((B * cap, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((B * cap, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda"))
           for _ in layers]
    kvs = [H.make_kv(k, v, cap, B) for k, v in kvt]
    b = H.Batch(np.arange(B + 1), [cached] * B, np.arange(B))
    emb = (torch.randn((B, D), device="cuda") * 0.02).to(torch.bfloat16)
    logits = torch.empty((B, K * V), dtype=torch.float32, device="cuda")
    frame = dev(np.full(B, 20, np.int32))
    seen, done = torch.zeros((B, K), dtype=torch.uint8, device="cuda"), torch.zeros(B, dtype=torch.uint8,
                                                                                      device="cuda")
    codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    ws = torch.empty(H.hr_decode_workspace_bytes(dims, H.HR_BF16, B), dtype=torch.uint8, device="cuda")

    def call():
        H.hr_decode_step(dims, layers, b, emb, kvs, shared["final"], shared["head"], K, V, m.bos_id, m.eoc_id,
                         logits, frame, seen, done, codes, None, 0, shared["cb"], emb, ws)
    sec = time_events(call, reps, warm=1)
    kv_bytes = len(layers) * B * (cached + 1) * m.n_kv_heads * m.head_dim * 2 * 2
    weight_bytes = sum(sum(t.numel() * t.element_size() for t in dl.values()) for dl in dev_layers)
    bytes_ = weight_bytes + K * V * D * 2 + kv_bytes
    del kvt
    return {"B": B, "cached_rows": cached, "ms_per_step": round(sec * 1e3, 4),
            "frames_per_s": round(B / sec, 1), "bytes": int(bytes_), "roofline": hbm(bytes_, sec)}


def codebook_steps(H, m, shared, B=64, reps=100):
    """The delayed-codebook step at B streams, 8 x 1026, bf16 logits."""
    import torch
    import synth
    from gpu_util import dev, dev_bf16
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    logits = dev_bf16(synth.codebook_logits(B, K, V, 0, m.eoc_id))
    st = synth.codebook_state(B, K)
    frame, seen, done = dev(st["frame"]), dev(st["eoc_seen"]), dev(st["done"])
    codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")

    def call():
        H.hr_codebook_step(B, K, V, m.bos_id, m.eoc_id, logits, frame, seen, done, codes, None, 0, shared["cb"], D,
                           emb)
    sec = time_events(call, reps)
    bytes_ = B * (K * V * 2 + K * D * 2 + D * 2 + K * 4 + K + 8)
    return {"B": B, "us_per_step": round(sec * 1e6, 2), "bytes": int(bytes_), "roofline": hbm(bytes_, sec)}


def codebook_policy_steps(H, m, shared, B=64, reps=100):
    """The sampled codebook step at B streams, 8 x 1026, bf16 logits, serving
    settings (temperature 1, top-k 50, top-p 0.95, per-stream Philox keys), with
    the EOC cascade and the repeated-code guard (limit 64) on.  The streams' frame
    counters advance every call, so each call draws fresh noise."""
    import torch
    import synth
    from gpu_util import dev, dev_bf16
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    logits = dev_bf16(synth.codebook_logits(B, K, V, 0, m.eoc_id))
    st = synth.codebook_state(B, K)
    frame, seen, done = dev(st["frame"]), dev(st["eoc_seen"]), dev(st["done"])
    codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
    sp = synth.sampling_settings(B, serving=True)
    end = dev(np.full(B, -1, np.int32))
    last = dev(np.full((B, K), -1, np.int32))
    run = dev(np.zeros(B, np.int32))
    pol = H.make_policy(temperature=dev(sp["temperature"]), top_k=dev(sp["top_k"]), top_p=dev(sp["top_p"]),
                        seed=dev(sp["seed"].view(np.int64)), eoc_cascade=True, repeat_limit=64, end_frame=end,
                        last_codes=last, repeat_run=run)

    def call():
        H.hr_codebook_step_policy(B, K, V, m.bos_id, m.eoc_id, logits, frame, seen, done, codes, None, 0,
                                  shared["cb"], D, emb, pol)
    sec = time_events(call, reps)
    bytes_ = B * (K * V * 2 + K * D * 2 + D * 2 + K * 4 + K + 8 + 16 + K * 8 + 8)
    return {"B": B, "us_per_step": round(sec * 1e6, 2), "bytes": int(bytes_), "roofline": hbm(bytes_, sec),
            "settings": "T 1, top-k 50, top-p 0.95, EOC cascade, repeat guard 64"}


def hbm_sweep(H, m, shared, reps=10):
    """The memory-bound kernels where their bytes outgrow launch latency:
    RMSNorm (6 B per element: fp32 in, fp16 out), the fused residual add +
    RMSNorm (14 B per element), q/k norm + RoPE + KV write
    (36.9 KB per token: fp32 QKV row in, fp16 q and bf16 K/V out), codebook
    step (62.5 KB per stream)."""
    import torch
    from model_util import dims_of
    out = {}
    D = m.hidden
    for T in (4096, 65536):
        h = torch.randn((T, D), device="cuda")
        x = torch.empty((T, D), dtype=torch.float16, device="cuda")
        sec = time_events(lambda: H.hr_rmsnorm(h, T, D, shared["final"], m.rms_eps, x), reps)
        out[f"rmsnorm_T{T}"] = {"us": round(sec * 1e6, 2), "roofline": hbm(6 * T * D, sec)}
        del h, x
    # fused residual add + RMSNorm: h and one split's partial in, h and x out (14 B per element)
    for T in (4096, 16384):
        h = torch.randn((T, D), device="cuda")
        part = torch.randn((1, T, D), device="cuda")
        x = torch.empty((T, D), dtype=torch.float16, device="cuda")
        sec = time_events(lambda: H.hr_residual_rmsnorm(h, part, 1, T, D, shared["final"], m.rms_eps, x), reps)
        out[f"residual_rmsnorm_T{T}"] = {"us": round(sec * 1e6, 2), "roofline": hbm(14 * T * D, sec)}
        del h, part, x
    for T in (4096, 32768):
        dims = dims_of(H, m, True, 1)
        qkv = torch.randn((T, m.qkv_rows), device="cuda") * 0.5
        q = torch.empty((T, m.attn_width), dtype=torch.float16, device="cuda")
        kc = torch.empty((T, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        b = H.Batch([0, T], [0], [0])
        kv = H.make_kv(kc, vc, T, 1)
        qn = shared["final"][:m.head_dim]
        sec = time_events(lambda: H.hr_qknorm_rope_kv(dims, b, qkv, qn, qn, q, kv), reps)
        bytes_ = T * (m.qkv_rows * 4 + m.attn_width * 2 + 2 * m.n_kv_heads * m.head_dim * 2)
        out[f"qknorm_rope_kv_T{T}"] = {"us": round(sec * 1e6, 2), "roofline": hbm(bytes_, sec)}
        del qkv, q, kc, vc
    for B in (4096, 16384):
        r = codebook_steps(H, m, shared, B=B, reps=reps)
        out[f"codebook_B{B}"] = {"us": r["us_per_step"], "roofline": r["roofline"]}
    r = codebook_policy_steps(H, m, shared, B=4096, reps=reps)
    out["codebook_sampled_B4096"] = {"us": r["us_per_step"], "roofline": r["roofline"]}
    return out


def cpu_baseline(m, P, host_layers, shared_host):
    """The float64 oracle, timed on the host cores on a bounded sample of the
    same workloads: the P-token prefill of the whole stack (every layer given
    in ``host_layers``, scaled to m.n_layers if fewer) plus final norm and head
    on the last row (the headline value, prompt tok/s); the same at P = 13
    (ms per prompt); and the delayed-codebook step on 64 streams x 8 x 1026
    bf16 logits (us per step).  Weight widening is outside the timed parts."""
    import synth
    from oracle import codebook as oc
    from oracle import prefill as op
    from oracle import numerics as nx
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    wh = nx.bf16_to_f64(shared_host["head"])
    wf = nx.bf16_to_f64(shared_host["final"])

    def stack_time(P_):
        ids = synth.prompt_ids(m, P_)
        h = nx.bf16_to_f64(synth.embed_rows(m, ids))
        b = {"cu_seqlens": [0, P_], "start_pos": [0], "cache_slot": [0], "capacity": P_}
        t_layers = 0.0
        for bits in host_layers:
            lw = op.widen_layer(bits)
            kc, vc = op.new_cache(m, 1, P_)
            t0 = time.perf_counter()
            h = op.prefill_layer(m, lw, b, h, kc, vc)
            t_layers += time.perf_counter() - t0
            del lw
        t0 = time.perf_counter()
        z = op.final_norm(m, h, wf)
        op.head_logits(z[-1:], wh, m.n_codebooks, m.cb_vocab)
        t_head = time.perf_counter() - t0
        return t_layers / len(host_layers) * m.n_layers + t_head, t_layers

    per_prompt, t_l = stack_time(P)
    per13, t13 = stack_time(13)
    # codebook step, B = 64
    B, K, V = 64, m.n_codebooks, m.cb_vocab
    logits = nx.bf16_to_f64(synth.codebook_logits(B, K, V, 0, m.eoc_id))
    st = synth.codebook_state(B, K)
    cb32 = nx.bf16_to_f32(shared_host["cb"])
    t0 = time.perf_counter()
    oc.codebook_step(logits, st["frame"].copy(), st["eoc_seen"].copy(), st["done"].copy(), m.bos_id, m.eoc_id, cb32)
    t_cb = time.perf_counter() - t0
    n = len(host_layers)
    return {"value": round(P / per_prompt, 3), "unit": "prompt tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {m.n_layers} layers of the P={P} prefill in float64 ({t_l:.1f} s of layer compute), "
                      f"scaled x{m.n_layers / n:g}, plus final norm + head on the last row; the same at P=13 "
                      f"({t13:.1f} s); one codebook step of 64 streams x {K} x {V}",
            "ms_per_prompt": round(per_prompt * 1e3, 1),
            "p13_ms_per_prompt": round(per13 * 1e3, 1),
            "codebook_b64_us_per_step": round(t_cb * 1e6, 1)}


def probe(H, m, layers, shared, dev_layers):
    """Launches for the counter runs (rocprofv3 --pmc): three P=512 stack
    steps, three P=13 steps (the weight-streaming projections), the FP8
    layer, the memory-bound kernels at sweep sizes and a 256 MiB device copy
    whose counter readings calibrate the byte counters."""
    import torch
    for P in (512, 13):
        st = Stack(H, m, P, dev_layers, layers, shared)
        for _ in range(3):
            st.step()
        torch.cuda.synchronize()
        del st
    fp8_layer(H, m, dev_layers[0], reps=2)
    sweep = hbm_sweep(H, m, shared, reps=2)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    return sweep


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each step as a captured HIP graph")
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--headline-only", action="store_true", help="skip the other measurement rows")
    ap.add_argument("--weights", choices=("packed", "bf16"), default="packed",
                    help="timed path: bf16 weights packed once by hr_pack_weight (the same products) or as stored")
    ap.add_argument("--probe", action="store_true",
                    help="only the launches the rocprofv3 counter runs read (no timing line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path is built and "
              f"measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import codebook_decode_amd.hr as H
    from gpu_util import dev_bf16
    H.lib()
    m = synth.QWEN3_4B.with_layers(args.layers)
    log(f"device {torch.cuda.get_device_name(0)}")
    t0 = time.time()
    shared = {"embed": dev_bf16(synth.embed_table(m)), "final": dev_bf16(synth.final_norm(m)),
              "head": dev_bf16(synth.head_weight(m)), "cb": dev_bf16(synth.codebook_embed(m))}
    log(f"embedding / head tables ready in {time.time() - t0:.1f} s")
    packed = args.weights == "packed"
    dev_layers, pk_layers, layers, host_layers = build_model(H, m, m.n_layers,
                                                             keep_host=not args.no_cpu and not args.probe,
                                                             packed=packed)
    wtype = H.HR_F16_PACKED if packed else H.HR_BF16
    run_layers = pk_layers if packed else dev_layers      # device weights of the timed path
    if args.probe:
        probe(H, m, layers, shared, dev_layers)
        log("probe launches done")
        return

    # headline: P = 512
    P = 512
    st512 = Stack(H, m, P, dev_layers, layers, shared)
    log("timing P=512 steps")
    sec = time_steps(st512.step, args.steps, args.warmup, args.graph)
    tok_s = P / sec
    log(f"P=512: {sec * 1e3:.3f} ms/step, {tok_s:.0f} tok/s")
    # P = 13 latency
    st13 = Stack(H, m, 13, dev_layers, layers, shared)
    sec13 = time_steps(st13.step, args.steps, args.warmup, args.graph)
    log(f"P=13: {sec13 * 1e3:.3f} ms/prompt")
    weight_bytes = sum(sum(t.numel() * t.element_size() for t in dl.values()) for dl in dev_layers)
    head_bytes = shared["head"].numel() * 2
    # dominant kernel at P=512: the gate/up GEMM (49% of the layer's FLOPs)
    fns = gemm_gu_launches(H, m, P, run_layers, wtype)
    t_gu = time_kernel_events(fns)
    flops_gu = 2.0 * P * m.hidden * 2 * m.ffn
    achieved = flops_gu / t_gu / 1e12
    layer_flops = 2.0 * P * m.hidden * (m.qkv_rows + 2 * m.ffn) + 2.0 * P * m.attn_width * m.hidden \
        + 2.0 * P * m.ffn * m.hidden
    attn_flops = 2.0 * 2 * m.n_q_heads * m.head_dim * (P * (P + 1) / 2)
    stack_flops = m.n_layers * (layer_flops + attn_flops)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "prompt tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "numerics": ("bf16 weights (" + ("packed once to fp16 by hr_pack_weight: the same values, bit-identical "
                     "results to the unpacked path" if packed else "as stored") + "); fp16 activations into fp16 "
                     "MFMAs with fp32 accumulation; fp32 residual; bf16 KV cache"),
        "data": "synthetic (seeded N(0,0.02) weights, uniform token ids)",
        "config": {"workload": f"stack{m.n_layers}_d2560_p512: Qwen3-style 4B decoder stack, {m.n_layers} layers, "
                               "hidden 2560, 32/8 heads x 128, SwiGLU 9728, single prompt P=512, causal, "
                               "KV cache 2048, audio head 8 x 1026 + delayed-codebook step",
                   "prompt_len": P, "layers": m.n_layers, "graph": bool(args.graph), "weights": args.weights},
        "roofline": {"bound": "mfma", "kernel": f"gemm_tiled SwiGLU (gate/up 512 x 19456 x 2560, {args.weights} weights)",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic(),
                     "avg_launch_us": round(t_gu * 1e6, 2)},
        "stack_p512": {"tflops_effective": round(stack_flops / sec / 1e12, 2),
                       "mfma_frac": round(stack_flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "p13": {"ms_per_prompt": round(sec13 * 1e3, 4),
                "roofline": {"bound": "hbm", "achieved": round((weight_bytes + head_bytes) / sec13 / 1e9, 1),
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round((weight_bytes + head_bytes) / sec13 / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes_per_prompt": int(weight_bytes + head_bytes)},
                "pages_context_ms": 6.82},
    }
    # the other measurement rows: P=128, one layer at P=6/13 (weights streamed
    # from HBM), FP8 layer, varlen batch, codebook step, memory-bound sweep
    if m.n_layers == 36 and not args.headline_only:
        log("timing P=128, the single layer, FP8, varlen, codebook and the HBM sweep")
        st128 = Stack(H, m, 128, dev_layers, layers, shared)
        sec128 = time_steps(st128.step, args.steps, args.warmup, args.graph)
        del st128
        out["p128"] = {"ms_per_prompt": round(sec128 * 1e3, 4),
                       "roofline": hbm(weight_bytes + head_bytes, sec128)}
        out["layer_d2560"] = layer_rotated(H, m, run_layers, wtype=wtype)
        if packed:
            # the same stack on the weights as stored (bf16, converted in registers)
            st_b = Stack(H, m, P, dev_layers, [H.make_layer(dl) for dl in dev_layers], shared)
            sec_b = time_steps(st_b.step, args.steps, args.warmup, args.graph)
            del st_b
            out["stack_p512_bf16_layout"] = {"ms_per_step": round(sec_b * 1e3, 4), "tok_s": round(P / sec_b, 1)}
        out["fp8_layer"] = fp8_layer(H, m, dev_layers[0])
        out["mxfp4_layer"] = mxfp4_layer(H, m, dev_layers[0])
        out["varlen32"] = varlen_batch(H, m, layers, shared)
        out["codebook_b64"] = codebook_steps(H, m, shared)
        out["codebook_sampled_b64"] = codebook_policy_steps(H, m, shared)
        log("timing decode steps (B=64 over 512 cached rows, B=16 and B=1 over 2047)")
        out["decode_b64"] = decode_steps(H, m, dev_layers, layers, shared, 64, 512)
        out["decode_b16"] = decode_steps(H, m, dev_layers, layers, shared, 16, 2047)
        out["decode_b1"] = decode_steps(H, m, dev_layers, layers, shared, 1, 2047)
        out["hbm_sweep"] = hbm_sweep(H, m, shared)
        torch.cuda.synchronize()
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(m, P, host_layers,
                                           {"head": synth.head_weight(m), "final": synth.final_norm(m),
                                            "cb": synth.codebook_embed(m)})
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
