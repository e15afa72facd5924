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


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def build_model(H, m, n_layers, keep_host=False):
    """Seeded weights of every layer, uploaded; returns device tensors, structs
    and (keep_host) the host bf16 bit patterns for the CPU oracle."""
    import torch
    import synth
    from model_util import upload_layer
    layers, dev_layers, host = [], [], []
    t0 = time.time()
    for l in range(n_layers):
        bits = synth.layer_tensors(m, l)
        dl = upload_layer(bits)
        dev_layers.append(dl)
        layers.append(H.make_layer(dl))
        if keep_host:
            host.append(bits)
    torch.cuda.synchronize()
    log(f"weights of {n_layers} layers drawn and uploaded in {time.time() - t0:.1f} s")
    return dev_layers, layers, host


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


def gemm_gu_launches(H, m, P, dev_layers):
    """The gate/up + SwiGLU GEMM of the P-row prefill, one launch per layer's weights."""
    import torch
    x = torch.randn((P, m.hidden), device="cuda").to(torch.bfloat16)
    out = torch.empty((P, m.ffn), dtype=torch.bfloat16, device="cuda")
    fns = []
    for dl in dev_layers:
        w = dl["w_gu"]
        fns.append(lambda w=w: H.hr_linear(x, w, None, 1.0, H.HR_BF16, P, 2 * m.ffn, m.hidden, H.HR_EPI_SWIGLU,
                                           out))
    return fns


def cpu_baseline(m, P, host_layers):
    """The float64 oracle on the P-token prefill of the whole stack (every layer
    given in ``host_layers``, scaled to m.n_layers if fewer), plus final norm
    and head on the last row.  Weight widening is outside the timed part."""
    import synth
    from oracle import prefill as op
    from oracle import numerics as nx
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    ids = synth.prompt_ids(m, P)
    h = nx.bf16_to_f64(synth.embed_rows(m, ids))
    b = {"cu_seqlens": [0, P], "start_pos": [0], "cache_slot": [0], "capacity": P}
    t_layers = 0.0
    n_sample_layers = len(host_layers)
    for bits in host_layers:
        lw = op.widen_layer(bits)
        kc, vc = op.new_cache(m, 1, P)
        t0 = time.perf_counter()
        h = op.prefill_layer(m, lw, b, h, kc, vc)
        t_layers += time.perf_counter() - t0
        del lw
    wh = nx.bf16_to_f64(synth.head_weight(m))
    wf = nx.bf16_to_f64(synth.final_norm(m))
    t0 = time.perf_counter()
    z = op.final_norm(m, h, wf)
    op.head_logits(z[-1:], wh, m.n_codebooks, m.cb_vocab)
    t_head = time.perf_counter() - t0
    per_prompt = t_layers / n_sample_layers * m.n_layers + t_head
    return {"value": round(P / per_prompt, 3), "unit": "prompt tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_sample_layers} of {m.n_layers} layers of the P={P} prefill in float64 "
                      f"({t_layers:.1f} s of layer compute), scaled x{m.n_layers / n_sample_layers:g}, "
                      f"plus final norm + head on the last row",
            "ms_per_prompt": round(per_prompt * 1e3, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each step as a captured HIP graph")
    ap.add_argument("--layers", type=int, default=36)
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
    dev_layers, layers, host_layers = build_model(H, m, m.n_layers, keep_host=not args.no_cpu)

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
    fns = gemm_gu_launches(H, m, P, dev_layers)
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
        "data": "synthetic (seeded N(0,0.02) weights, uniform token ids)",
        "config": {"workload": f"stack{m.n_layers}_d2560_p512: Qwen3-style 4B decoder stack, {m.n_layers} layers, "
                               "hidden 2560, 32/8 heads x 128, SwiGLU 9728, single prompt P=512, causal, "
                               "KV cache 2048, audio head 8 x 1026 + delayed-codebook step",
                   "prompt_len": P, "layers": m.n_layers, "graph": bool(args.graph)},
        "roofline": {"bound": "mfma", "kernel": "gemm_tiled SwiGLU (gate/up 512 x 19456 x 2560)",
                     "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
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
    if not args.no_cpu:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(m, P, host_layers)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
