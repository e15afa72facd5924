"""hr_decode_step_noalloc (scratch in the library's fixed device array) against
hr_decode_step (scratch in a caller workspace) through the C ABI: two decode
steps in a row on a 2-layer 4B-shape stack, the second with fewer streams, on
identical copies of every input; logits, codes, codebook-embedding sums,
stream state and both layers' KV caches must be equal bit for bit (the two run
the same kernels, and every reduction has a fixed order).  A batch whose
scratch exceeds the array is refused on the host before any launch."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def _step_inputs(m, B, cap, seed):
    """Seeded decode-step inputs for B streams: cache rows [0, start) of each
    slot, the new rows' input embeddings, the codebook-step state."""
    rng = np.random.default_rng(seed)
    starts = rng.integers(1, cap - 1, B).astype(np.int32)
    shape = (B * cap, m.n_kv_heads, m.head_dim)
    caches = []
    for l in range(m.n_layers):
        kb = np.full(shape, 0x7FC0, np.uint16)
        vb = np.full(shape, 0x7FC0, np.uint16)
        for s, sp in enumerate(starts):
            kb[s * cap: s * cap + sp] = synth.normal_bf16((int(sp),) + shape[1:], (61, seed, l, 0, s), 1.0)
            vb[s * cap: s * cap + sp] = synth.normal_bf16((int(sp),) + shape[1:], (61, seed, l, 1, s), 1.0)
        caches.append((kb, vb))
    x = synth.embed_rows(m, synth.prompt_ids(m, B, seq=500 + seed))
    frame = rng.integers(0, 12, B).astype(np.int32)
    return starts, caches, x, frame


def _run(H, fn_name, m, layers, shared, B, cap, inputs):
    """One decode step through the named entry on fresh device copies."""
    import torch
    from gpu_util import bits_of, dev, dev_bf16
    from model_util import dims_of
    starts, caches, x, frame0 = inputs
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    dims = dims_of(H, m, True, m.n_layers)
    kvt = [(dev_bf16(kb), dev_bf16(vb)) for kb, vb in caches]
    kvs = [H.make_kv(k, v, cap, B) for k, v in kvt]
    b = H.Batch(np.arange(B + 1), starts, np.arange(B))
    emb_in = dev_bf16(x)
    logits = torch.full((B, K * V), float("nan"), dtype=torch.float32, device="cuda")
    frame = dev(frame0.copy())
    seen = torch.zeros((B, K), dtype=torch.uint8, device="cuda")
    done = torch.zeros(B, dtype=torch.uint8, device="cuda")
    codes = torch.full((B, K), -1, dtype=torch.int32, device="cuda")
    emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
    args = (dims, layers, b, emb_in, kvs, shared["final"], shared["head"], K, V, m.bos_id, m.eoc_id, logits, frame,
            seen, done, codes, None, 0, shared["cb"], emb)
    if fn_name == "noalloc":
        H.hr_decode_step_noalloc(*args)
    else:
        ws = torch.empty(H.hr_decode_workspace_bytes(dims, H.HR_BF16, B), dtype=torch.uint8, device="cuda")
        H.hr_decode_step(*args, ws)
    torch.cuda.synchronize()
    out = {"logits": logits.cpu().numpy(), "codes": codes.cpu().numpy(), "emb": bits_of(emb),
           "frame": frame.cpu().numpy(), "seen": seen.cpu().numpy(), "done": done.cpu().numpy()}
    for l, (k, v) in enumerate(kvt):
        out[f"k{l}"], out[f"v{l}"] = bits_of(k), bits_of(v)
    return out


def test_noalloc_decode_matches_workspace_entry(H):
    from gpu_util import dev_bf16, log
    from model_util import upload_layer
    m = synth.QWEN3_4B.with_layers(2)
    cap = 300
    layers = [H.make_layer(upload_layer(synth.layer_tensors(m, l))) for l in range(m.n_layers)]
    shared = {"final": dev_bf16(synth.final_norm(m)), "head": dev_bf16(synth.head_weight(m)),
              "cb": dev_bf16(synth.codebook_embed(m))}
    for B, seed in ((8, 1), (3, 2)):          # the second call smaller than the first
        log(f"no-alloc decode step: B={B}")
        inputs = _step_inputs(m, B, cap, seed)
        ref = _run(H, "workspace", m, layers, shared, B, cap, inputs)
        got = _run(H, "noalloc", m, layers, shared, B, cap, inputs)
        assert np.all(np.isfinite(got["logits"]))
        for key in ref:
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"B={B}: {key}")


def test_noalloc_decode_refuses_oversized_batch(H):
    import torch
    from gpu_util import dev_bf16
    from model_util import dims_of, upload_layer
    m = synth.QWEN3_4B.with_layers(1)
    dims = dims_of(H, m, True, 1)
    B, cap = 200, 4
    need = H.hr_decode_workspace_bytes(dims, H.HR_BF16, B)
    assert need > H.hr_decode_noalloc_scratch_bytes(), need
    # properly sized buffers all the same, so no call here could reach past them
    K, V, D = m.n_codebooks, m.cb_vocab, m.hidden
    layer = H.make_layer(upload_layer(synth.layer_tensors(m, 0)))
    k = torch.zeros((B * cap, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    b = H.Batch(np.arange(B + 1), np.ones(B), np.arange(B))
    emb = torch.zeros((B, D), dtype=torch.bfloat16, device="cuda")
    logits = torch.zeros((B, K * V), dtype=torch.float32, device="cuda")
    frame = torch.zeros(B, dtype=torch.int32, device="cuda")
    seen = torch.zeros((B, K), dtype=torch.uint8, device="cuda")
    done = torch.zeros(B, dtype=torch.uint8, device="cuda")
    codes = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    fw, hw, cb = dev_bf16(synth.final_norm(m)), dev_bf16(synth.head_weight(m)), dev_bf16(synth.codebook_embed(m))
    with pytest.raises(H.HrError, match="HR_EWORKSPACE"):
        H.hr_decode_step_noalloc(dims, [layer], b, emb, [H.make_kv(k, v, cap, B)], fw, hw, K, V, m.bos_id, m.eoc_id,
                                 logits, frame, seen, done, codes, None, 0, cb, emb)
    torch.cuda.synchronize()
    assert int(frame.sum()) == 0 and int(codes.sum()) == 0      # nothing ran
