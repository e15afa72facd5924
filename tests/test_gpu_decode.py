"""Batched autoregressive decode on the GPU against the float64 oracle: one new
row per stream at its cached length, attention over the stream's cache rows,
the audio head and the delayed-codebook step.

* A 4B layer over four one-row streams whose caches already hold 460-1900
  rows (seeded values): 4 streams x 8 kv heads give 32 query blocks, the
  longest row spans 30 key tiles, so the layer splits the rows into key
  chunks and merges the partials.  Per-layer bf16 checks as for the prefill.
* The FP8 layer on the same kind of decode step (the attention output in
  e4m3), at the FP8 bar against the unquantised and the fake-quant oracle.
* hr_decode_step on the tiny model, three streams prefilled with different
  prompt lengths, six steps: each step's logits against the oracle's; the
  step inside hr_decode_step equal bit for bit to the oracle's step on the
  GPU's own logits (codes, state, embedding sums); codes equal to the
  oracle's free-running codes except where the oracle's top-2 margin is below
  1e-3 (the comparison stops at such a near-tie).
* hr_decode_step on two 4B layers over four streams with long seeded caches:
  logits at the bf16-band bar, the step bit-exact on the GPU's logits, codes
  equal to the oracle's except where its top-2 margin is below 1e-3.
"""
import numpy as np
import pytest

import synth
from oracle import codebook as oc
from oracle import numerics as nx
from oracle import prefill as op

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def seeded_prefix(m, starts, slots, cap, key):
    """bf16 bits of cache rows [0, start) of each slot (K and V), NaN elsewhere."""
    n_slots = max(slots) + 1
    shape = (n_slots * cap, m.n_kv_heads, m.head_dim)
    kb = np.full(shape, 0x7FC0, np.uint16)
    vb = np.full(shape, 0x7FC0, np.uint16)
    for s, (sp, slot) in enumerate(zip(starts, slots)):
        if sp == 0:
            continue
        rows = (sp, m.n_kv_heads, m.head_dim)
        kb[slot * cap: slot * cap + sp] = synth.normal_bf16(rows, key + (0, s), 1.0)
        vb[slot * cap: slot * cap + sp] = synth.normal_bf16(rows, key + (1, s), 1.0)
    return kb, vb


def caches_from_bits(kb, vb):
    """(gpu K, gpu V) bf16 tensors and (oracle K, oracle V) float64 arrays."""
    import torch
    gk = torch.from_numpy(kb.view(np.int16).copy()).to("cuda").view(torch.bfloat16)
    gv = torch.from_numpy(vb.view(np.int16).copy()).to("cuda").view(torch.bfloat16)
    return (gk, gv), (nx.bf16_to_f64(kb), nx.bf16_to_f64(vb))


def test_layer_decode_rows_over_long_caches(H):
    from gpu_util import log
    from test_gpu_layer import check_hidden, compare_caches, oracle_layer, run_gpu_layer
    m = synth.QWEN3_4B.with_layers(1)
    lens, starts, slots, cap = [1, 1, 1, 1], [1900, 700, 1200, 460], [0, 1, 2, 3], 2048
    log(f"decode rows over long caches: starts {starts}")
    bits = synth.layer_tensors(m, 0)
    kb, vb = seeded_prefix(m, starts, slots, cap, (77,))
    h0 = nx.bf16_to_f64(synth.embed_rows(m, synth.prompt_ids(m, 4, seq=5)))
    (gk, gv), (ok, ov) = caches_from_bits(kb, vb)
    hg, kcg, vcg = run_gpu_layer(H, m, bits, lens, starts, slots, cap, h0, caches=(gk, gv))
    hr, kcr, vcr = oracle_layer(m, bits, lens, starts, slots, cap, h0, caches=(ok, ov))
    check_hidden("hidden", hg, hr)
    compare_caches(kcg, vcg, kcr, vcr)


def test_layer_decode_fp8_rows_over_long_caches(H):
    """The FP8 layer on a decode step (one row per stream over seeded caches):
    the new rows' q/k norm, RoPE and K/V write inside the decode attention
    launch, its output quantised to e4m3 for the O projection.  Held to the FP8
    bar against the unquantised and the fake-quant oracle."""
    import torch
    from gpu_util import bits_of, cosine, log
    from model_util import fp8_pack, upload_layer
    from oracle import fp8 as of
    from test_gpu_layer import check_fp8, fp8_scales, oracle_layer, run_gpu_layer
    m = synth.QWEN3_4B.with_layers(1)
    lens, starts, slots, cap = [1, 1, 1, 1], [1900, 700, 1200, 460], [0, 1, 2, 3], 2048
    log(f"fp8 decode rows over long caches: starts {starts}")
    bits = synth.layer_tensors(m, 0)
    lw = op.widen_layer(bits)
    scales, = fp8_scales(m, [lw])
    kb, vb = seeded_prefix(m, starts, slots, cap, (78,))
    h0 = nx.bf16_to_f64(synth.embed_rows(m, synth.prompt_ids(m, 4, seq=6)))
    import codebook_decode_amd.hr as HH
    w8, ws = fp8_pack(HH, upload_layer(bits), m)
    torch.cuda.synchronize()
    (gk, gv), (ok, ov) = caches_from_bits(kb, vb)
    hg, kcg, vcg = run_gpu_layer(H, m, bits, lens, starts, slots, cap, h0, caches=(gk, gv),
                                 fp8=(scales, (w8, ws)))
    hr, kcr, vcr = oracle_layer(m, bits, lens, starts, slots, cap, h0, caches=(ok, ov))
    _, (fk, fv) = caches_from_bits(kb, vb)
    packed = of.pack_layer({k: v.astype(np.float32) for k, v in lw.items()})
    ob = {"cu_seqlens": np.arange(5), "start_pos": starts, "cache_slot": slots, "capacity": cap}
    hf = of.fp8_layer(m, lw, scales, packed, ob, h0, fk, fv, True, None)
    check_fp8("fp8 decode hidden", hg, hr, hf)
    rows = [sl * cap + sp for sp, sl in zip(starts, slots)]
    kgb = bits_of(kcg)
    ck = cosine(nx.bf16_to_f64(kgb[rows]), kcr[rows])
    log(f"  fp8 decode new K rows cos = {ck:.6f}")
    assert ck >= 0.998
    kgb[rows] = kb[rows]
    np.testing.assert_array_equal(kgb, kb)                  # no other row written


def _oracle_decode(m, lw_of, starts, slots, cap, x_rows, caches, wf, wh):
    """One decode step of the stack in the oracle: layers over the new rows,
    final norm, head.  caches: list of (kc, vc) float64, updated in place."""
    B = len(starts)
    b = {"cu_seqlens": np.arange(B + 1), "start_pos": starts, "cache_slot": slots, "capacity": cap}
    h = np.asarray(x_rows, dtype=np.float64)
    for l in range(m.n_layers):
        kc, vc = caches[l]
        h = op.prefill_layer(m, lw_of(l), b, h, kc, vc, True, None)
    z = op.final_norm(m, h, wf)
    return op.head_logits(z, wh, m.n_codebooks, m.cb_vocab)


def test_decode_step_tiny_batched(H):
    import torch
    from gpu_util import bits_of, dev, dev_bf16, log
    from model_util import dims_of, kv_cache, upload_layer, workspace
    from test_gpu_layer import check
    m = synth.TINY
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    lens, cap, steps = [5, 9, 6], 64, 6
    B = len(lens)
    slots = list(range(B))
    bits = synth.layer_tensors(m, 0)
    lw = op.widen_layer(bits)
    E, wf, wh, Ecb = synth.embed_table(m), synth.final_norm(m), synth.head_weight(m), synth.codebook_embed(m)
    dims = dims_of(H, m, True, 1)
    layer = H.make_layer(upload_layer(bits))
    kc, vc = kv_cache(m, B, cap)
    kv = H.make_kv(kc, vc, cap, B)
    okc, ovc = op.new_cache(m, B, cap)
    ids = np.concatenate([synth.prompt_ids(m, n, seq=20 + s) for s, n in enumerate(lens)])
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    # prefill of the three prompts and the first codebook step
    bp = H.Batch(cu, [0] * B, slots)
    h = torch.empty((T, D), dtype=torch.float32, device="cuda")
    logits = torch.empty((B, K * V), dtype=torch.float32, device="cuda")
    H.hr_prefill_stack(dims, [layer], bp, dev(ids), dev_bf16(E), m.vocab, None, [kv], dev_bf16(wf), dev_bf16(wh),
                       K, V, h, logits, workspace(H, dims, H.HR_BF16, T))
    ob = {"cu_seqlens": cu, "start_pos": [0] * B, "cache_slot": slots, "capacity": cap}
    _, _, olog = op.prefill_stack(m, lambda l: lw, ob, nx.bf16_to_f64(E[ids]), [(okc, ovc)],
                                  nx.bf16_to_f64(wf), nx.bf16_to_f64(wh))
    frame, seen, done = dev(np.zeros(B, np.int32)), dev(np.zeros((B, K), np.uint8)), dev(np.zeros(B, np.uint8))
    codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
    o_frame, o_seen, o_done = np.zeros(B, np.int32), np.zeros((B, K), np.uint8), np.zeros(B, np.uint8)
    Ecb32 = nx.bf16_to_f32(Ecb)
    dEcb = dev_bf16(Ecb)
    H.hr_codebook_step(B, K, V, m.bos_id, m.eoc_id, logits.view(B, K, V), frame, seen, done, codes, None, 0,
                       dEcb, D, emb)
    ocodes, oemb = oc.codebook_step(olog.astype(np.float64), o_frame, o_seen, o_done, m.bos_id, m.eoc_id, Ecb32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(codes.cpu().numpy(), ocodes)
    np.testing.assert_array_equal(bits_of(emb), oemb)
    # decode steps through hr_decode_step; emb is both this step's input and
    # the next step's output
    ws = torch.empty(H.hr_decode_workspace_bytes(dims, H.HR_BF16, B), dtype=torch.uint8, device="cuda")
    dwf, dwh = dev_bf16(wf), dev_bf16(wh)
    for t in range(steps):
        starts = [n + t for n in lens]
        bd = H.Batch(np.arange(B + 1), starts, slots)
        log(f"tiny decode step {t}: positions {starts}")
        g_state = (frame.cpu().numpy(), seen.cpu().numpy(), done.cpu().numpy())
        H.hr_decode_step(dims, [layer], bd, emb, [kv], dwf, dwh, K, V, m.bos_id, m.eoc_id, logits, frame, seen,
                         done, codes, None, 0, dEcb, emb, ws)
        check_step_on(logits.cpu().numpy().reshape(B, K, V), g_state, codes, emb, frame, seen, done, m, Ecb32)
        olog = _oracle_decode(m, lambda l: lw, starts, slots, cap, nx.bf16_to_f64(oemb), [(okc, ovc)],
                              nx.bf16_to_f64(wf), nx.bf16_to_f64(wh))
        margin = oc.top2_margin(olog)
        ocodes, oemb = oc.codebook_step(olog.astype(np.float64), o_frame, o_seen, o_done, m.bos_id, m.eoc_id,
                                        Ecb32)
        torch.cuda.synchronize()
        check(f"step {t} logits", logits.cpu().numpy().reshape(B, K, V), olog)
        gcodes = codes.cpu().numpy()
        diff = gcodes != ocodes
        if np.any(diff):
            assert np.all(margin[diff] < 1e-3), f"step {t}: codes differ outside the 1e-3 margin exemption"
            log(f"step {t}: codes differ on a near-tie; stopping the free-running comparison")
            return
        np.testing.assert_array_equal(bits_of(emb), oemb)
        np.testing.assert_array_equal(frame.cpu().numpy(), o_frame)
        np.testing.assert_array_equal(seen.cpu().numpy(), o_seen)
        np.testing.assert_array_equal(done.cpu().numpy(), o_done)


def test_decode_step_4b_two_layers_long_caches(H):
    import torch
    from gpu_util import bits_of, cosine, dev, dev_bf16, log, max_abs
    from model_util import dims_of, upload_layer
    m = synth.QWEN3_4B.with_layers(2)
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    starts, cap = [1000, 300, 600, 129], 1024
    B = len(starts)
    slots = list(range(B))
    log(f"4B 2-layer decode step: positions {starts}")
    bits = [synth.layer_tensors(m, l) for l in range(2)]
    lws = [op.widen_layer(b) for b in bits]
    layers = [H.make_layer(upload_layer(b)) for b in bits]
    wf, wh, Ecb = synth.final_norm(m), synth.head_weight(m), synth.codebook_embed(m)
    dims = dims_of(H, m, True, 2)
    gpu_caches, ora = [], []
    for l in range(2):
        kb, vb = seeded_prefix(m, starts, slots, cap, (78, l))
        g, o = caches_from_bits(kb, vb)
        gpu_caches.append(g)
        ora.append(o)
    kvs = [H.make_kv(k, v, cap, B) for k, v in gpu_caches]
    x_bits = synth.embed_rows(m, synth.prompt_ids(m, B, seq=9))
    x = dev_bf16(x_bits)
    frame0 = np.array([3, 10, 0, 20], np.int32)
    frame, seen, done = dev(frame0), dev(np.zeros((B, K), np.uint8)), dev(np.zeros(B, np.uint8))
    codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
    logits = torch.empty((B, K * V), dtype=torch.float32, device="cuda")
    ws = torch.empty(H.hr_decode_workspace_bytes(dims, H.HR_BF16, B), dtype=torch.uint8, device="cuda")
    bd = H.Batch(np.arange(B + 1), starts, slots)
    H.hr_decode_step(dims, layers, bd, x, kvs, dev_bf16(wf), dev_bf16(wh), K, V, m.bos_id, m.eoc_id, logits,
                     frame, seen, done, codes, None, 0, dev_bf16(Ecb), emb, ws)
    x64 = nx.bf16_to_f64(x_bits)
    olog = _oracle_decode(m, lambda l: lws[l], starts, slots, cap, x64, ora, nx.bf16_to_f64(wf),
                          nx.bf16_to_f64(wh))
    torch.cuda.synchronize()
    glog = logits.cpu().numpy().astype(np.float64).reshape(B, K, V)
    c, a = cosine(glog, olog), max_abs(glog, olog)
    log(f"  logits: cos={c:.7f} max_abs={a:.3g}")
    assert np.all(np.isfinite(glog))
    assert c >= 0.9999 and a <= 3e-2, (c, a)
    check_step_on(logits.cpu().numpy().reshape(B, K, V),
                  (frame0, np.zeros((B, K), np.uint8), np.zeros(B, np.uint8)), codes, emb, frame, seen, done, m,
                  nx.bf16_to_f32(Ecb))
    ocodes, oemb = oc.codebook_step(olog, frame0.copy(), np.zeros((B, K), np.uint8), np.zeros(B, np.uint8),
                                    m.bos_id, m.eoc_id, nx.bf16_to_f32(Ecb))
    gcodes = codes.cpu().numpy()
    margin = oc.top2_margin(olog)
    diff = gcodes != ocodes
    log(f"  codes equal on {int((~diff).sum())} of {diff.size}; smallest margin where different: "
        f"{float(margin[diff].min()) if diff.any() else None}")
    assert np.all(margin[diff] < 1e-3), "codes differ outside the 1e-3 margin exemption"
    same = ~diff.any(axis=1)
    np.testing.assert_array_equal(bits_of(emb)[same], oemb[same])
    np.testing.assert_array_equal(frame.cpu().numpy(), frame0 + 1)


def check_step_on(g_logits, g_state, codes, emb, frame, seen, done, m, Ecb32):
    """The codebook step a decode step ran on its own fp32 logits, bit for bit
    against the oracle's step on those logits from the same stream state."""
    from gpu_util import bits_of
    f0, s0, d0 = (np.array(a, copy=True) for a in g_state)
    ocodes, oemb = oc.codebook_step(g_logits, f0, s0, d0, m.bos_id, m.eoc_id, Ecb32)
    np.testing.assert_array_equal(codes.cpu().numpy(), ocodes)
    np.testing.assert_array_equal(bits_of(emb), oemb)
    np.testing.assert_array_equal(frame.cpu().numpy(), f0)
    np.testing.assert_array_equal(seen.cpu().numpy(), s0)
    np.testing.assert_array_equal(done.cpu().numpy(), d0)
