"""hr_prefill_layer / hr_prefill_stack against the same layer composed from the
step-level entry points of include/hr_ops.h (one call per step), on new tokens
every repetition.

Both run the same kernels in the same configuration, and every reduction is in
a fixed order (the residual projections' split-K partials are summed in split
order, no atomics), so hidden state and caches must be equal bit for bit: a
layer call that skipped, reordered or mis-addressed a step (a stale workspace
region, a cache row written to the wrong slot) or a result that changed from
run to run fails.  The one exception is a decode step over long caches, where
the layer entry splits the attention into key chunks (its workspace holds the
partials) and the composed steps run it unsplit: there the bar is the per-layer
bf16-band bar (cosine >= 0.9999, max |diff| <= 3e-2), and the cache rows must
still be equal bit for bit.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

REPS = 3


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


@pytest.fixture(scope="module")
def layers(H):
    from model_util import upload_layer
    m = synth.QWEN3_4B
    return m, [upload_layer(synth.layer_tensors(m, l)) for l in range(2)]


def composed_layer(H, m, dims, batch, dl, h, kv, T, fused_short=False):
    """One layer from the step-level entries (activations fp16, QKV rows
    fp32).  ``fused_short``: steps A3 + A4 through hr_qknorm_rope_attention,
    the launch the layer entries take for prompts of at most 32 rows from
    position 0 (unless every sequence has one row: a decode step)."""
    import torch
    D, F, A, NQKV = m.hidden, m.ffn, m.attn_width, m.qkv_rows
    ws_o = H.linear_ws(H.HR_BF16, T, D, A, H.HR_EPI_RESIDUAL)
    ws_d = H.linear_ws(H.HR_BF16, T, D, F, H.HR_EPI_RESIDUAL)
    hf = dict(dtype=torch.float16, device="cuda")
    x, qkv = torch.empty((T, D), **hf), torch.empty((T, NQKV), dtype=torch.float32, device="cuda")
    q, attn, act = torch.empty((T, A), **hf), torch.empty((T, A), **hf), torch.empty((T, F), **hf)
    H.hr_rmsnorm(h, T, D, dl["in_norm"], m.rms_eps, x)
    H.hr_linear(x, dl["w_qkv"], None, 1.0, H.HR_BF16, T, NQKV, D, H.HR_EPI_F32, qkv)
    if fused_short:
        H.hr_qknorm_rope_attention(dims, batch, qkv, dl["q_norm"], dl["k_norm"], kv, attn)
    else:
        H.hr_qknorm_rope_kv(dims, batch, qkv, dl["q_norm"], dl["k_norm"], q, kv)
        H.hr_attention(dims, batch, q, kv, attn)
    H.hr_linear(attn, dl["w_o"], None, 1.0, H.HR_BF16, T, D, A, H.HR_EPI_RESIDUAL, h, ws=ws_o)
    H.hr_rmsnorm(h, T, D, dl["post_norm"], m.rms_eps, x)
    H.hr_linear(x, dl["w_gu"], None, 1.0, H.HR_BF16, T, 2 * F, D, H.HR_EPI_SWIGLU, act)
    H.hr_linear(act, dl["w_down"], None, 1.0, H.HR_BF16, T, D, F, H.HR_EPI_RESIDUAL, h, ws=ws_d)


def close(name, got, ref, exact=True):
    from gpu_util import cosine, log, max_abs
    c, a = cosine(got, ref), max_abs(got, ref)
    log(f"  {name}: cos={c:.8f} max_abs={a:.3g}")
    assert np.all(np.isfinite(got)), name
    if exact:
        np.testing.assert_array_equal(np.asarray(got), np.asarray(ref), err_msg=name)
    else:
        assert c >= 0.9999 and a <= 3e-2, (name, c, a)


@pytest.mark.parametrize("T", [1, 13, 40, 64, 512])
def test_layer_matches_composed_steps(H, layers, T):
    """hr_prefill_layer at T tokens (one sequence), REPS times on new tokens."""
    import torch
    from gpu_util import bits_of, dev, log
    from model_util import dims_of, kv_cache, workspace
    m, dls = layers
    cap = max(64, T)
    dims = dims_of(H, m, True, 1)
    layer = H.make_layer(dls[0])
    b = H.Batch([0, T], [0], [0])
    ws = workspace(H, dims, H.HR_BF16, T)
    for r in range(REPS):
        log(f"layer T={T} repetition {r}")
        ids = synth.prompt_ids(m, T, seq=100 + r)
        h0 = synth.embed_rows(m, ids)
        h_init = synth.bf16_bits_to_f32(h0)
        hf, hc = dev(h_init.copy()), dev(h_init.copy())
        kf, vf = kv_cache(m, 1, cap)
        kc, vc = kv_cache(m, 1, cap)
        H.hr_prefill_layer(dims, layer, b, hf, H.make_kv(kf, vf, cap, 1), ws)
        composed_layer(H, m, dims, b, dls[0], hc, H.make_kv(kc, vc, cap, 1), T, fused_short=1 < T <= 32)
        torch.cuda.synchronize()
        # from 385 to 1024 causal rows the layer's attention reads the fp16 copies
        # its fused QKV launch writes (hr_attention_f16's kernel): the same values
        # in another summation order, so the hidden meets the bar instead of the bits
        close("hidden", hf.cpu().numpy(), hc.cpu().numpy(), exact=not 384 < T <= 1024)
        close("K cache", kf[:T].float().cpu().numpy(), kc[:T].float().cpu().numpy())
        close("V cache", vf[:T].float().cpu().numpy(), vc[:T].float().cpu().numpy())
        assert np.all(bits_of(kf)[T:] == 0x7FC0), "stray cache write"


def test_stack_two_layers_matches_composed_steps(H, layers):
    """hr_prefill_stack over two layers at 13 tokens, REPS times."""
    import torch
    from gpu_util import dev, dev_bf16, log
    from model_util import dims_of, kv_cache, workspace
    m, dls = layers
    T, cap = 13, 64
    dims = dims_of(H, m, True, 2)
    E = dev_bf16(synth.embed_table(m))
    wf = dev_bf16(synth.final_norm(m))
    b = H.Batch([0, T], [0], [0])
    ws = workspace(H, dims, H.HR_BF16, T)
    dims1 = dims_of(H, m, True, 1)
    for r in range(REPS):
        log(f"2-layer stack repetition {r}")
        ids = synth.prompt_ids(m, T, seq=200 + r)
        h = torch.empty((T, m.hidden), dtype=torch.float32, device="cuda")
        caches = [kv_cache(m, 1, cap) for _ in range(2)]
        H.hr_prefill_stack(dims, [H.make_layer(d) for d in dls], b, dev(ids), E, m.vocab, None,
                           [H.make_kv(k, v, cap, 1) for k, v in caches], wf, None, 0, 0, h, None, ws)
        hc = dev(synth.bf16_bits_to_f32(synth.embed_rows(m, ids)))
        for l in range(2):
            kc, vc = kv_cache(m, 1, cap)
            composed_layer(H, m, dims1, b, dls[l], hc, H.make_kv(kc, vc, cap, 1), T, fused_short=True)
        torch.cuda.synchronize()
        close("hidden after 2 layers", h.cpu().numpy(), hc.cpu().numpy())


@pytest.mark.parametrize("starts,slots", [
    ([37, 700, 1500, 2046], [1, 3, 0, 2]),      # split into key chunks (the layer's workspace)
    ([0, 5, 63, 64], [0, 1, 2, 3]),             # one chunk each; a stream at position 0
])
def test_decode_layer_matches_composed_steps(H, layers, starts, slots):
    """A decode step (one row per stream over seeded caches): the layer, which
    norms and rotates q / k and writes the new K/V row inside the decode
    attention launch, against the composed steps (hr_qknorm_rope_kv, then
    hr_attention).  The new cache rows must hold the same bits, every other
    row must be untouched, the hidden within the bar above."""
    import torch
    from gpu_util import bits_of, dev, dev_bf16, log
    from model_util import dims_of, workspace
    m, dls = layers
    B, cap = len(starts), 2048
    dims = dims_of(H, m, True, 1)
    layer = H.make_layer(dls[0])
    b = H.Batch(np.arange(B + 1), starts, slots)
    ws = workspace(H, dims, H.HR_BF16, B)
    shape = (B * cap, m.n_kv_heads, m.head_dim)
    kb = np.full(shape, 0x7FC0, np.uint16)
    vb = np.full(shape, 0x7FC0, np.uint16)
    for s, (sp, slot) in enumerate(zip(starts, slots)):
        if sp:
            kb[slot * cap: slot * cap + sp] = synth.normal_bf16((sp,) + shape[1:], (60, 0, s), 1.0)
            vb[slot * cap: slot * cap + sp] = synth.normal_bf16((sp,) + shape[1:], (60, 1, s), 1.0)
    for r in range(REPS):
        log(f"decode layer starts={starts} repetition {r}")
        h_init = synth.bf16_bits_to_f32(synth.embed_rows(m, synth.prompt_ids(m, B, seq=300 + r)))
        hf, hc = dev(h_init.copy()), dev(h_init.copy())
        kf, vf, kc, vc = dev_bf16(kb), dev_bf16(vb), dev_bf16(kb), dev_bf16(vb)
        H.hr_prefill_layer(dims, layer, b, hf, H.make_kv(kf, vf, cap, B), ws)
        composed_layer(H, m, dims, b, dls[0], hc, H.make_kv(kc, vc, cap, B), B)
        torch.cuda.synchronize()
        close("hidden", hf.cpu().numpy(), hc.cpu().numpy(), exact=starts[-1] < 64)
        np.testing.assert_array_equal(bits_of(kf), bits_of(kc))
        np.testing.assert_array_equal(bits_of(vf), bits_of(vc))
        new_rows = [slot * cap + sp for sp, slot in zip(starts, slots)]
        kfb = bits_of(kf)
        assert not np.any(kfb[new_rows] == 0x7FC0), "new K rows not written"
        kfb[new_rows] = kb[new_rows]
        np.testing.assert_array_equal(kfb, kb)      # nothing else written
