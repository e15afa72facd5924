"""hr_prefill_stack captured in a HIP graph (torch.cuda.CUDAGraph on a side
stream) and replayed: every replay, with eager work and synchronisations of
the program in between, must give what the eager call gives, bit for bit:
the library records kernels only (no memset nodes) and every reduction runs in
a fixed order (split-K partials summed in split order), so hidden state,
logits and every layer's KV cache repeat exactly; no row past the prompt may
be written.
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


@pytest.mark.parametrize("P", [13, 512])
def test_stack_graph_replays_match_eager(H, P):
    import torch
    from gpu_util import bits_of, dev, dev_bf16, log, max_abs
    from model_util import dims_of, kv_cache, upload_layer, workspace
    m = synth.QWEN3_4B
    n_layers = 2
    dims = dims_of(H, m, True, n_layers)
    layers = [H.make_layer(upload_layer(synth.layer_tensors(m, l))) for l in range(n_layers)]
    E, wf, wh = dev_bf16(synth.embed_table(m)), dev_bf16(synth.final_norm(m)), dev_bf16(synth.head_weight(m))
    cap = 1024
    caches = [kv_cache(m, 1, cap) for _ in range(n_layers)]
    kvs = [H.make_kv(k, v, cap, 1) for k, v in caches]
    b = H.Batch([0, P], [0], [0])
    ids = dev(synth.prompt_ids(m, P, seq=400))
    K, V = m.n_codebooks, m.cb_vocab
    h = torch.empty((P, m.hidden), dtype=torch.float32, device="cuda")
    logits = torch.empty((1, K * V), dtype=torch.float32, device="cuda")
    ws = workspace(H, dims, H.HR_BF16, P)

    def call():
        H.hr_prefill_stack(dims, layers, b, ids, E, m.vocab, None, kvs, wf, wh, K, V, h, logits, ws)

    log(f"graph stack P={P}: eager reference")
    call()
    torch.cuda.synchronize()
    h_ref, l_ref = h.cpu().numpy().copy(), logits.cpu().numpy().copy()
    kv_ref = [(bits_of(k).copy(), bits_of(v).copy()) for k, v in caches]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(3):
        h.fill_(float("nan"))
        logits.fill_(float("nan"))
        for k, v in caches:
            k.fill_(float("nan"))
            v.fill_(float("nan"))
        scratch.add_(1.0)                      # eager work of the program between replays
        torch.cuda.synchronize()
        log(f"graph stack P={P}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        hg, lg = h.cpu().numpy(), logits.cpu().numpy()
        assert np.all(np.isfinite(hg)) and np.all(np.isfinite(lg)), r
        log(f"  replay {r}: hidden max diff {max_abs(hg, h_ref):.3g}; logits max diff {max_abs(lg, l_ref):.3g}")
        np.testing.assert_array_equal(hg, h_ref)
        np.testing.assert_array_equal(lg, l_ref)
        for (k, v), (kr, vr) in zip(caches, kv_ref):
            for t, ref in ((k, kr), (v, vr)):
                b_ = bits_of(t)
                np.testing.assert_array_equal(b_[:P], ref[:P])
                assert np.all(b_[P:] == 0x7FC0)
