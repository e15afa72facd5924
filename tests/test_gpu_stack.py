"""Full-size stacks on the GPU against the float64 oracle.

Per layer (teacher-forced): GPU layer l runs on the oracle's output of layer
l - 1 (inputs flow oracle -> GPU only) and is held to the bf16-band bars
(hidden and written K/V rows: cosine >= 0.9999, max |err| <= 3e-2).

Head ids at the per-layer bar: the GPU's last layer (on the oracle's h_34)
and the GPU's head give argmax ids equal to the oracle's except where the
oracle's top-2 margin is below 1e-3.

Free running: hr_prefill_stack with the audio head from the token ids.
  * final hidden and logits: cosine >= 0.9999 against the oracle stack;
  * hr_codebook_step on the GPU's own logits equals the oracle's step on
    those same logits bit for bit (codes, state, embedding sums);
  * argmax ids: 36 layers of 16-bit rounding move the logits by a few 1e-2
    (logged), more than the 1e-3 margin exemption presumes, so a free-running
    id may differ from the oracle's only where the oracle's top-2 margin is
    below twice that row's largest logit error (the gap such an error can
    close); every difference is logged.

Workloads: the 36-layer 4B stack at P = 13 and P = 512 (the two headline
prompts), and the 32-prompt varlen batch (lengths uniform on [6, 256], packed,
one 256-row cache slot per prompt; every sequence checked).
"""
import time

import numpy as np
import pytest

import synth
from oracle import codebook as oc
from oracle import numerics as nx
from oracle import prefill as op

pytestmark = pytest.mark.gpu

FREE_COS_MIN = 0.9999
ID_MARGIN = 1e-3


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


@pytest.fixture(scope="module")
def model_36(H):
    """Seeded weights of the 36 layers, uploaded once (7.3 GB), host bits kept."""
    from gpu_util import dev_bf16, log
    from model_util import upload_layer
    m = synth.QWEN3_4B
    t0 = time.time()
    host, devl = [], []
    for l in range(m.n_layers):
        bits = synth.layer_tensors(m, l)
        host.append(bits)
        devl.append(upload_layer(bits))
    shared = {"embed": dev_bf16(synth.embed_table(m)), "final": synth.final_norm(m), "head": synth.head_weight(m),
              "cb": synth.codebook_embed(m)}
    shared["d_final"], shared["d_head"] = dev_bf16(shared["final"]), dev_bf16(shared["head"])
    shared["d_cb"] = dev_bf16(shared["cb"])
    log(f"36-layer model drawn and uploaded in {time.time() - t0:.1f} s")
    return m, host, devl, shared


def check_ids(g_log, o_log, exempt=ID_MARGIN):
    """Argmax ids per codebook: equal to the oracle's except where the oracle's
    top-2 margin is below ``exempt`` (1e-3, or per-row values)."""
    from gpu_util import log
    g_ids, o_ids = g_log.argmax(-1), o_log.argmax(-1)
    margin = oc.top2_margin(o_log)
    diff = g_ids != o_ids
    log(f"  ids gpu {g_ids.tolist()} oracle {o_ids.tolist()} min margin {float(margin.min()):.4g}"
        + (f"; differ at codebooks {np.nonzero(diff)[0].tolist()} (margins {margin[diff].tolist()})"
           if diff.any() else ""))
    assert np.all(~diff | (margin < exempt)), (g_ids, o_ids, margin, exempt)


def check_step_on_gpu_logits(H, m, sh, g_log_dev, n):
    """hr_codebook_step on the GPU's fp32 logits against the oracle's step on
    the same logits: bit-exact codes, frame / EOC / done state and embedding
    sums (streams at frames 0 and 9, so both the BOS fill and emitted codes
    occur)."""
    import torch
    from gpu_util import bits_of, dev
    K, V = m.n_codebooks, m.cb_vocab
    frame0 = (np.arange(n) % 2 * 9).astype(np.int32)
    frame, seen, done = dev(frame0), dev(np.zeros((n, K), np.uint8)), dev(np.zeros(n, np.uint8))
    codes = torch.empty((n, K), dtype=torch.int32, device="cuda")
    emb = torch.empty((n, m.hidden), dtype=torch.bfloat16, device="cuda")
    H.hr_codebook_step(n, K, V, m.bos_id, m.eoc_id, g_log_dev.view(n, K, V), frame, seen, done, codes, None, 0,
                       sh["d_cb"], m.hidden, emb)
    torch.cuda.synchronize()
    logits = g_log_dev.cpu().numpy().reshape(n, K, V)
    o_frame, o_seen, o_done = frame0.copy(), np.zeros((n, K), np.uint8), np.zeros(n, np.uint8)
    ocodes, oemb = oc.codebook_step(logits, o_frame, o_seen, o_done, m.bos_id, m.eoc_id, nx.bf16_to_f32(sh["cb"]))
    np.testing.assert_array_equal(codes.cpu().numpy(), ocodes)
    np.testing.assert_array_equal(frame.cpu().numpy(), o_frame)
    np.testing.assert_array_equal(seen.cpu().numpy(), o_seen)
    np.testing.assert_array_equal(done.cpu().numpy(), o_done)
    np.testing.assert_array_equal(bits_of(emb), oemb)


def _teacher_forced_and_free(H, model_36, lens, cap, tag):
    """Per-layer teacher-forced checks over every layer, then the free-running
    stack with the head, for a packed batch of prompts from position 0."""
    import torch
    from gpu_util import cosine, dev, log, max_abs
    from model_util import dims_of, kv_cache, workspace
    from test_gpu_layer import check_hidden, compare_caches
    m, host, devl, sh = model_36
    lens = [int(x) for x in lens]
    n = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    ids = np.concatenate([synth.prompt_ids(m, L, seq=s) for s, L in enumerate(lens)]) if n > 1 \
        else synth.prompt_ids(m, lens[0])
    h_prev = nx.bf16_to_f64(synth.embed_rows(m, ids))
    ob = {"cu_seqlens": cu, "start_pos": np.zeros(n, int), "cache_slot": np.arange(n), "capacity": cap}
    dims1 = dims_of(H, m, True, 1)
    b = H.Batch(cu, np.zeros(n), np.arange(n))
    ws = workspace(H, dims1, H.HR_BF16, T)
    worst = 0.0
    h_last_gpu = None
    for l in range(m.n_layers):
        lw = op.widen_layer(host[l])
        okc, ovc = op.new_cache(m, n, cap)
        h_ref = op.prefill_layer(m, lw, ob, h_prev, okc, ovc)
        kc, vc = kv_cache(m, n, cap)
        h = dev(h_prev.astype(np.float32))
        H.hr_prefill_layer(dims1, H.make_layer(devl[l]), b, h, H.make_kv(kc, vc, cap, n), ws)
        torch.cuda.synchronize()
        log(f"{tag} layer {l}")
        g = h.cpu().numpy().astype(np.float64)
        check_hidden(f"{tag} layer {l} hidden", g, h_ref)
        compare_caches(kc, vc, okc, ovc)
        worst = max(worst, max_abs(g, h_ref))
        h_prev = h_ref
        if l == m.n_layers - 1:
            h_last_gpu = h
        del kc, vc, okc, ovc
    log(f"{tag}: worst per-layer max abs {worst:.4f}")
    hL = h_prev                       # the oracle stack run free (teacher forcing fed it only itself)
    K, V = m.n_codebooks, m.cb_vocab
    z = op.final_norm(m, hL, nx.bf16_to_f64(sh["final"]))
    olog = op.head_logits(z[cu[1:] - 1], nx.bf16_to_f64(sh["head"]), K, V)

    # the head on the GPU's last layer (fed the oracle's h_34): ids at the 1e-3 exemption
    tlog = torch.empty((n, K * V), dtype=torch.float32, device="cuda")
    hws = torch.empty(H.hr_head_workspace_bytes(n, m.hidden), dtype=torch.uint8, device="cuda")
    H.hr_head_logits(h_last_gpu, b, m.hidden, sh["d_final"], m.rms_eps, sh["d_head"], K, V, tlog, hws)
    torch.cuda.synchronize()
    t_log = tlog.cpu().numpy().astype(np.float64).reshape(n, K, V)
    log(f"{tag} teacher-forced head: logits max_abs={max_abs(t_log, olog):.3g}")
    for s in range(n):
        check_ids(t_log[s], olog[s])

    dims = dims_of(H, m, True)
    kvs = [kv_cache(m, n, cap, poison=False) for _ in range(m.n_layers)]
    h_out = torch.empty((T, m.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((n, K * V), dtype=torch.float32, device="cuda")
    H.hr_prefill_stack(dims, [H.make_layer(d) for d in devl], b, dev(ids), sh["embed"], m.vocab, None,
                       [H.make_kv(k, v, cap, n) for k, v in kvs], sh["d_final"], sh["d_head"], K, V, h_out, logits,
                       workspace(H, dims, H.HR_BF16, T))
    torch.cuda.synchronize()
    del kvs
    g_h = h_out.cpu().numpy().astype(np.float64)
    g_log = logits.cpu().numpy().astype(np.float64).reshape(n, K, V)
    assert np.all(np.isfinite(g_h)) and np.all(np.isfinite(g_log))
    for s in range(n):
        rows = slice(cu[s], cu[s + 1])
        c_h, c_l = cosine(g_h[rows], hL[rows]), cosine(g_log[s], olog[s])
        log(f"{tag} free-running seq {s} (len {lens[s]}): h_L cos={c_h:.7f} max_abs={max_abs(g_h[rows], hL[rows]):.3g}"
            f" (|h_L| max {np.abs(hL[rows]).max():.1f}); logits cos={c_l:.7f} "
            f"max_abs={max_abs(g_log[s], olog[s]):.3g}")
        assert c_h >= FREE_COS_MIN, (s, c_h)
        assert c_l >= FREE_COS_MIN, (s, c_l)
        row_err = np.max(np.abs(g_log[s] - olog[s]), axis=-1)
        check_ids(g_log[s], olog[s], exempt=np.maximum(ID_MARGIN, 2.0 * row_err))
    check_step_on_gpu_logits(H, m, sh, logits, n)


@pytest.mark.timeout(900)
def test_stack36_p13(H, model_36):
    _teacher_forced_and_free(H, model_36, [13], 2048, "P=13")


@pytest.mark.timeout(900)
def test_stack36_p512(H, model_36):
    _teacher_forced_and_free(H, model_36, [512], 2048, "P=512")


@pytest.mark.timeout(1200)
def test_varlen32_stack36(H, model_36):
    m = model_36[0]
    w = synth.workloads()["varlen32_stack36_d2560"]
    _teacher_forced_and_free(H, model_36, w.prompt_lens, w.capacity, "varlen32")


@pytest.mark.timeout(600)
def test_stack36_p512_packed_equals_bf16(H, model_36):
    """The 36-layer stack with its weights packed by hr_pack_weight (the
    format the benchmark times) gives the bf16 stack's hidden states, logits
    and KV caches bit for bit."""
    import torch
    from gpu_util import dev, log
    from model_util import dims_of, kv_cache, workspace
    m, host, devl, sh = model_36
    shapes = {"w_qkv": (m.qkv_rows, m.hidden), "w_o": (m.hidden, m.attn_width), "w_gu": (2 * m.ffn, m.hidden),
              "w_down": (m.hidden, m.ffn)}
    P, cap = 512, 1024
    K, V = m.n_codebooks, m.cb_vocab
    ids = dev(synth.prompt_ids(m, P))
    b = H.Batch([0, P], [0], [0])
    dims = dims_of(H, m, True)
    res = []
    for packed in (False, True):
        if packed:
            dls = [H.pack_layer_weights(d, shapes) for d in devl]
            layers = [H.make_layer(d, H.HR_F16_PACKED) for d in dls]
            wtype = H.HR_F16_PACKED
        else:
            dls, layers, wtype = devl, [H.make_layer(d) for d in devl], H.HR_BF16
        kvs = [kv_cache(m, 1, cap, poison=False) for _ in range(m.n_layers)]
        h_out = torch.empty((P, m.hidden), dtype=torch.float32, device="cuda")
        logits = torch.empty((1, K * V), dtype=torch.float32, device="cuda")
        H.hr_prefill_stack(dims, layers, b, ids, sh["embed"], m.vocab, None, [H.make_kv(k, v, cap, 1) for k, v in kvs],
                           sh["d_final"], sh["d_head"], K, V, h_out, logits, workspace(H, dims, wtype, P))
        torch.cuda.synchronize()
        log(f"stack P=512 packed={packed} done")
        res.append((h_out.cpu().numpy(), logits.cpu().numpy(),
                    kvs[-1][0].cpu().view(torch.int16).numpy(), kvs[-1][1].cpu().view(torch.int16).numpy()))
        del kvs
        if packed:
            del dls, layers
    for a, b_ in zip(res[0], res[1]):
        np.testing.assert_array_equal(a, b_)

