"""hr_prefill_layer / hr_prefill_stack on the GPU against the float64 oracle.

bf16 weights (the band computes with fp16 activations), per layer, for the
hidden state and every written K/V cache row, against the exact float64
oracle: cosine >= 0.9999 and max |err| <= 3e-2.  Measured values are logged.
Cache rows outside the batch stay NaN.
FP8: the GPU's cosine against the unquantised layer must be no worse (minus
1e-3) than the oracle's fake-quant layer's (same scales, same packed weights:
the accuracy of the method itself), and the GPU stays within cosine 0.998 of
that fake-quant layer (the two round different near-ties to E4M3), 1 - cos
growing by at most 0.002 per layer over a stack.
Codebook ids: exact, except where the oracle's top-2 logit margin is < 1e-3."""
import numpy as np
import pytest

import synth
from oracle import codebook as oc
from oracle import fp8 as of
from oracle import numerics as nx
from oracle import prefill as op

pytestmark = pytest.mark.gpu

COS_MIN, ABS_MAX = 0.9999, 3e-2


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def check(name, got, ref, cos_min=COS_MIN, abs_max=ABS_MAX):
    from gpu_util import cosine, log, max_abs
    c, a = cosine(got, ref), max_abs(got, ref)
    log(f"  {name}: cos={c:.7f} max_abs={a:.3g}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    assert c >= cos_min, f"{name}: cosine {c}"
    assert a <= abs_max, f"{name}: max abs {a}"


def check_hidden(name, got, exact):
    """The bf16-band bars of the module docstring."""
    check(name, got, exact)


def run_gpu_layer(H, m, bits, lens, starts, slots, cap, h0, causal=True, used=None, caches=None,
                  fp8=None):
    import torch
    from gpu_util import dev
    from model_util import dims_of, kv_cache, upload_layer, workspace
    n_slots = max(slots) + 1
    kc, vc = caches if caches is not None else kv_cache(m, n_slots, cap)
    dl = upload_layer(bits)
    dims = dims_of(H, m, causal, 1)
    if fp8 is None:
        layer = H.make_layer(dl)
        wtype = H.HR_BF16
    else:
        scales, (w8, ws) = fp8
        layer = H.make_layer(w8, H.HR_FP8_E4M3, scales, ws)
        wtype = H.HR_FP8_E4M3
    b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), starts, slots, used)
    h = dev(np.ascontiguousarray(h0, dtype=np.float32))
    ws_ = workspace(H, dims, wtype, sum(lens))
    H.hr_prefill_layer(dims, layer, b, h, H.make_kv(kc, vc, cap, n_slots), ws_)
    torch.cuda.synchronize()
    return h.cpu().numpy().astype(np.float64), kc, vc


def oracle_layer(m, bits, lens, starts, slots, cap, h0, causal=True, used=None, caches=None):
    n_slots = max(slots) + 1
    kc, vc = caches if caches is not None else op.new_cache(m, n_slots, cap)
    b = {"cu_seqlens": np.concatenate([[0], np.cumsum(lens)]), "start_pos": starts, "cache_slot": slots,
         "capacity": cap}
    h = op.prefill_layer(m, op.widen_layer(bits), b, h0, kc, vc, causal, used)
    return h, kc, vc


def compare_caches(kc_gpu, vc_gpu, kc_ref, vc_ref):
    from gpu_util import BF16_NAN, bits_of
    kb, vb = bits_of(kc_gpu), bits_of(vc_gpu)
    written = ~np.isnan(kc_ref[:, 0, 0])
    check("K cache", nx.bf16_to_f64(kb[written]), kc_ref[written])
    check("V cache", nx.bf16_to_f64(vb[written]), vc_ref[written])
    assert np.all(kb[~written] == BF16_NAN) and np.all(vb[~written] == BF16_NAN), "stray cache write"


CASES = [
    ("tiny_d256_p6", synth.TINY, [6], [0], [0], 64),
    ("layer_d2560_p6", synth.QWEN3_4B, [6], [0], [0], 2048),
    ("layer_d2560_p13", synth.QWEN3_4B, [13], [0], [0], 2048),
    ("layer_d2560_varlen_t200", synth.QWEN3_4B, [100, 37, 63], [0, 0, 0], [1, 2, 0], 128),
    # 17-64 and 65-128 rows: the small-M tiles of every projection (down at K 9728)
    ("layer_d2560_p40", synth.QWEN3_4B, [40], [0], [0], 64),
    ("layer_d2560_p128", synth.QWEN3_4B, [128], [0], [0], 128),
    # the P = 512 prefill of the throughput measurement (256 x 256 gate/up tiles,
    # two wave groups per attention block)
    ("layer_d2560_p512", synth.QWEN3_4B, [512], [0], [0], 512),
    # above 1024 rows: the large-M tiles (varlen batches)
    ("layer_d2560_varlen_t1100", synth.QWEN3_4B, [600, 500], [0, 0], [0, 1], 600),
    # 385-1024 causal rows from position 0: the attention over the fp16 K/V
    # copies of the fused QKV launch, three sequences at batch rows 0, 296, 464
    # (multiples of 8); then a batch starting a sequence at row 300, which
    # keeps the cache kernel
    ("layer_d2560_varlen_t600_f16", synth.QWEN3_4B, [296, 168, 136], [0, 0, 0], [2, 0, 1], 304),
    ("layer_d2560_varlen_t429", synth.QWEN3_4B, [300, 129], [0, 0], [1, 0], 304),
]


@pytest.mark.parametrize("name,m,lens,starts,slots,cap", CASES, ids=[c[0] for c in CASES])
def test_layer_bf16(H, name, m, lens, starts, slots, cap):
    from gpu_util import log
    log(f"layer bf16 {name}")
    bits = synth.layer_tensors(m, 0)
    ids = np.concatenate([synth.prompt_ids(m, n, seq=s) for s, n in enumerate(lens)])
    h0 = nx.bf16_to_f64(synth.embed_rows(m, ids))
    hg, kcg, vcg = run_gpu_layer(H, m, bits, lens, starts, slots, cap, h0)
    hr, kcr, vcr = oracle_layer(m, bits, lens, starts, slots, cap, h0)
    check_hidden("hidden", hg, hr)
    compare_caches(kcg, vcg, kcr, vcr)


def test_layer_prefill_then_continuation(H):
    """10 prompt tokens, then 3 more at start_pos 10 reading the cache the first
    call wrote (the decode path: same call, start_pos > 0)."""
    from gpu_util import log
    from model_util import kv_cache
    log("layer continuation 10 + 3")
    m, cap = synth.QWEN3_4B, 64
    bits = synth.layer_tensors(m, 0)
    ids = synth.prompt_ids(m, 13)
    h0 = nx.bf16_to_f64(synth.embed_rows(m, ids))
    caches = kv_cache(m, 1, cap)
    ocaches = op.new_cache(m, 1, cap)
    g1, *_ = run_gpu_layer(H, m, bits, [10], [0], [0], cap, h0[:10], caches=caches)
    g2, kcg, vcg = run_gpu_layer(H, m, bits, [3], [10], [0], cap, h0[10:], caches=caches)
    r1, *_ = oracle_layer(m, bits, [10], [0], [0], cap, h0[:10], caches=ocaches)
    r2, kcr, vcr = oracle_layer(m, bits, [3], [10], [0], cap, h0[10:], caches=ocaches)
    check_hidden("hidden", np.concatenate([g1, g2]), np.concatenate([r1, r2]))
    compare_caches(kcg, vcg, kcr, vcr)


FP8_CASES = [
    # name, used rows P, rows, causal
    ("fp8_p512_pad544_noncausal", 512, 544, False),   # tiled GEMMs
    ("fp8_p40_pad48_noncausal", 40, 48, False),       # small-batch (skinny) projections
    ("fp8_p13_causal", 13, 13, True),
]


def fp8_scales(m, lws):
    """Static activation scales of consecutive layers from the fixed 32-token
    calibration prompt (layer l calibrated on the unquantised output of l-1)."""
    h = nx.bf16_to_f64(synth.embed_rows(m, synth.calibration_ids(m, 32)))
    out = []
    for lw in lws:
        out.append(of.calibrate(m, lw, h))
        kc, vc = op.new_cache(m, 1, 32)
        h = op.prefill_layer(m, lw, {"cu_seqlens": [0, 32], "start_pos": [0], "cache_slot": [0], "capacity": 32},
                             h, kc, vc, False, [32])
    return out


def check_fp8(name, got, exact, fake, n_layers=1):
    """FP8 bars: no less accurate than the method (fake-quant oracle vs
    unquantised, minus 1e-3), and within 1 - cos <= 0.002 per layer of the
    fake-quant oracle: each layer's E4M3 roundings of near-ties are taken on
    fp32 values on the GPU and on float64 ones in the oracle, and the
    disagreements of consecutive layers add up (to first order, in 1 - cos)."""
    from gpu_util import cosine, log
    c, cf, c_method = cosine(got, exact), cosine(got, fake), cosine(fake, exact)
    log(f"  {name} cos: vs fake-quant oracle {cf:.6f}; vs unquantised {c:.6f} "
        f"(fake-quant oracle vs unquantised {c_method:.6f})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    assert cf >= 1.0 - 0.002 * n_layers, f"{name}: cosine vs fake-quant {cf}"
    assert c >= c_method - 1e-3, f"{name}: cosine vs unquantised {c} < method's {c_method}"


@pytest.mark.parametrize("name,P,rows,causal", FP8_CASES, ids=[c[0] for c in FP8_CASES])
def test_layer_fp8(H, name, P, rows, causal):
    """FP8 layer of the 4B shape: `rows` rows, the first P used (non-causal over
    the used keys) or all causal; static activation scales from the fixed
    32-token calibration prompt; per-output-channel E4M3 weights packed on the
    device."""
    import torch
    from gpu_util import bits_of, cosine, log
    from model_util import fp8_pack, upload_layer
    m = synth.QWEN3_4B
    cap = rows
    log(f"layer {name}")
    bits = synth.layer_tensors(m, 0)
    lw = op.widen_layer(bits)
    scales, = fp8_scales(m, [lw])
    log(f"fp8 layer scales {scales}")
    ids = synth.prompt_ids(m, P)
    h0 = np.zeros((rows, m.hidden))
    h0[:P] = nx.bf16_to_f64(synth.embed_rows(m, ids))
    import codebook_decode_amd.hr as HH
    dl = upload_layer(bits)
    w8, ws = fp8_pack(HH, dl, m)
    torch.cuda.synchronize()
    # the device packing equals the oracle's packing, bit for bit
    s_ref, c_ref = of.weight_scales_e4m3(nx.bf16_to_f32(bits["w_o"]))
    np.testing.assert_array_equal(ws["o"].cpu().numpy(), s_ref)
    np.testing.assert_array_equal(nx.e4m3_decode(w8["w_o"].cpu().numpy()), nx.e4m3_decode(c_ref))
    used = None if causal else [P]
    hg, kcg, vcg = run_gpu_layer(H, m, bits, [rows], [0], [0], cap, h0, causal=causal, used=used,
                                 fp8=(scales, (w8, ws)))
    hr, kcr, vcr = oracle_layer(m, bits, [rows], [0], [0], cap, h0, causal=causal, used=used)
    packed = of.pack_layer({k: v.astype(np.float32) for k, v in lw.items()})
    fkc, fvc = op.new_cache(m, 1, cap)
    ob = {"cu_seqlens": [0, rows], "start_pos": [0], "cache_slot": [0], "capacity": cap}
    hf = of.fp8_layer(m, lw, scales, packed, ob, h0, fkc, fvc, causal, used)
    check_fp8("fp8 hidden", hg[:P], hr[:P], hf[:P])
    kb = bits_of(kcg)
    assert np.all(kb[P:] == 0x7FC0)                         # pad rows never written
    ck = cosine(nx.bf16_to_f64(kb[:P]), kcr[:P])
    log(f"  fp8 K cache cos = {ck:.6f}")
    assert ck >= 0.998


def test_stack_fp8_two_layers_small(H):
    """Two FP8 layers of the 4B shape through hr_prefill_stack at 13 tokens:
    the second layer's input norm (with its own activation scale) is computed
    inside the first layer's down projection on this path."""
    import torch
    from gpu_util import dev, dev_bf16, log
    from model_util import dims_of, fp8_pack, kv_cache, upload_layer, workspace
    m, P, cap = synth.QWEN3_4B, 13, 64
    log("fp8 stack 2 layers P=13")
    bits = [synth.layer_tensors(m, l) for l in range(2)]
    lws = [op.widen_layer(b) for b in bits]
    scales = fp8_scales(m, lws)
    import codebook_decode_amd.hr as HH
    layers, keep = [], []
    for b, sc in zip(bits, scales):
        w8, ws = fp8_pack(HH, upload_layer(b), m)
        keep.append((w8, ws))
        layers.append(H.make_layer(w8, H.HR_FP8_E4M3, sc, ws))
    caches = [kv_cache(m, 1, cap) for _ in range(2)]
    kvs = [H.make_kv(kc, vc, cap, 1) for kc, vc in caches]
    E = synth.embed_table(m)
    ids = synth.prompt_ids(m, P)
    dims = dims_of(H, m, True, 2)
    h = torch.empty((P, m.hidden), dtype=torch.float32, device="cuda")
    ws_ = workspace(H, dims, H.HR_FP8_E4M3, P)
    H.hr_prefill_stack(dims, layers, H.Batch([0, P], [0], [0]), dev(ids), dev_bf16(E), m.vocab, None, kvs,
                       dev_bf16(synth.final_norm(m)), None, 0, 0, h, None, ws_)
    torch.cuda.synchronize()
    hg = h.cpu().numpy().astype(np.float64)
    ob = {"cu_seqlens": [0, P], "start_pos": [0], "cache_slot": [0], "capacity": cap}
    he = hf = nx.bf16_to_f64(E[ids])
    for lw, sc in zip(lws, scales):
        kc, vc = op.new_cache(m, 1, cap)
        he = op.prefill_layer(m, lw, ob, he, kc, vc, True, None)
        kc, vc = op.new_cache(m, 1, cap)
        packed = of.pack_layer({k: v.astype(np.float32) for k, v in lw.items()})
        hf = of.fp8_layer(m, lw, sc, packed, ob, hf, kc, vc, True, None)
    check_fp8("fp8 2-layer hidden", hg, he, hf, n_layers=2)


def test_stack_tiny_prefill_head_and_decode_frames(H):
    """The tiny model end to end: P=6 prefill through hr_prefill_stack with the
    audio head, then 8 frames of (codebook step -> P=1 prefill of the summed
    codebook embedding at start_pos 6+t -> head)."""
    import torch
    from gpu_util import bits_of, dev, dev_bf16, log
    from model_util import dims_of, kv_cache, upload_layer, workspace
    m, P, cap, frames = synth.TINY, 6, 64, 8
    K, V = m.n_codebooks, m.cb_vocab
    bits = synth.layer_tensors(m, 0)
    dl = upload_layer(bits)
    E = synth.embed_table(m)
    wf, wh, Ecb = synth.final_norm(m), synth.head_weight(m), synth.codebook_embed(m)
    dE, dwf, dwh, dEcb = dev_bf16(E), dev_bf16(wf), dev_bf16(wh), dev_bf16(Ecb)
    ids = synth.prompt_ids(m, P)
    dims = dims_of(H, m, True, 1)
    layer = H.make_layer(dl)
    kc, vc = kv_cache(m, 1, cap)
    kv = H.make_kv(kc, vc, cap, 1)
    lw = op.widen_layer(bits)
    okc, ovc = op.new_cache(m, 1, cap)
    # prefill
    b = H.Batch([0, P], [0], [0])
    h = torch.empty((P, m.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((1, K * V), dtype=torch.float32, device="cuda")
    ws = workspace(H, dims, H.HR_BF16, P)
    log("tiny stack prefill P=6")
    H.hr_prefill_stack(dims, [layer], b, dev(ids), dE, m.vocab, None, [kv], dwf, dwh, K, V, h, logits, ws)
    ob = {"cu_seqlens": [0, P], "start_pos": [0], "cache_slot": [0], "capacity": cap}
    oh, oz, olog = op.prefill_stack(m, lambda l: lw, ob, nx.bf16_to_f64(E[ids]), [(okc, ovc)],
                                    nx.bf16_to_f64(wf), nx.bf16_to_f64(wh))
    torch.cuda.synchronize()
    check("prefill hidden", h.cpu().numpy(), oh)
    check("prefill logits", logits.cpu().numpy().reshape(1, K, V), olog)
    # decode frames
    frame = dev(np.zeros(1, np.int32))
    seen, done = dev(np.zeros((1, K), np.uint8)), dev(np.zeros(1, np.uint8))
    codes = torch.empty((1, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((1, m.hidden), dtype=torch.bfloat16, device="cuda")
    o_frame, o_seen, o_done = np.zeros(1, np.int32), np.zeros((1, K), np.uint8), np.zeros(1, np.uint8)
    Ecb32 = nx.bf16_to_f32(Ecb)
    for t in range(frames):
        margin = oc.top2_margin(olog)[0]
        log(f"frame {t}: oracle top-2 margins {np.round(margin, 4).tolist()}")
        H.hr_codebook_step(1, K, V, m.bos_id, m.eoc_id, logits.view(1, K, V), frame, seen, done, codes, None, 0,
                           dEcb, m.hidden, emb)
        ocodes, oemb = oc.codebook_step(olog.astype(np.float64), o_frame, o_seen, o_done, m.bos_id, m.eoc_id,
                                        Ecb32)
        torch.cuda.synchronize()
        gcodes = codes.cpu().numpy()
        exempt = margin < 1e-3
        if np.any(gcodes[0] != ocodes[0]):
            assert np.all(exempt[gcodes[0] != ocodes[0]]), f"frame {t}: ids differ outside the margin exemption"
            log(f"frame {t}: ids differ on a near-tie; stopping the free-running comparison")
            return
        np.testing.assert_array_equal(bits_of(emb), oemb)
        # next token: the summed codebook embedding at position P + t
        b1 = H.Batch([0, 1], [P + t], [0])
        H.hr_prefill_stack(dims, [layer], b1, None, None, 0, emb, [kv], dwf, dwh, K, V, h[:1], logits,
                           workspace(H, dims, H.HR_BF16, 1))
        ob1 = {"cu_seqlens": [0, 1], "start_pos": [P + t], "cache_slot": [0], "capacity": cap}
        oh1, _, olog = op.prefill_stack(m, lambda l: lw, ob1, nx.bf16_to_f64(oemb), [(okc, ovc)],
                                        nx.bf16_to_f64(wf), nx.bf16_to_f64(wh))
        torch.cuda.synchronize()
        check(f"frame {t} hidden", h[:1].cpu().numpy(), oh1)
        check(f"frame {t} logits", logits.cpu().numpy().reshape(1, K, V), olog)
