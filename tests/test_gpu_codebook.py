"""hr_codebook_step on the GPU: bit-exact against the hand-derived golden cases
and against the oracle on the batched workload (64 streams, 8 x 1026, 16 steps,
bf16 logits with EOC forced top-1 in 5% of rows), plus fp32 logits."""
import json
import os

import numpy as np
import pytest

import synth
from oracle import codebook as oc
from oracle import numerics as nx

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "codebook_cases.json")


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def run_gpu_steps(H, logits_list, frame, seen, done, E_bits, V, bos, eoc, max_frames, f32=False):
    import torch
    from gpu_util import dev, dev_bf16, bits_of
    B, K, _ = logits_list[0].shape
    D = E_bits.shape[1]
    d_frame, d_seen, d_done = dev(frame.copy()), dev(seen.copy()), dev(done.copy())
    d_aligned = dev(np.full((B, max_frames, K), -1, np.int32))
    d_codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
    d_emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
    d_E = dev_bf16(E_bits)
    out = []
    for lg in logits_list:
        d_lg = dev(lg) if f32 else dev_bf16(lg)
        H.hr_codebook_step(B, K, V, bos, eoc, d_lg, d_frame, d_seen, d_done, d_codes, d_aligned, max_frames,
                           d_E, D, d_emb)
        torch.cuda.synchronize()
        out.append((d_codes.cpu().numpy().copy(), bits_of(d_emb).copy()))
    return out, d_frame.cpu().numpy(), d_seen.cpu().numpy(), d_done.cpu().numpy(), d_aligned.cpu().numpy()


def test_golden_cases_bit_exact(H):
    from gpu_util import log
    g = json.load(open(GOLD))
    K, V = g["K"], g["V"]
    D = 8   # rows E[r] = [r, 0.5, 0, ...]: emb[0:2] = [sum of rows, 0.5 K]
    E = np.zeros((K * V, D), np.float32)
    E[:, 0] = np.arange(K * V)
    E[:, 1] = 0.5
    E_bits = nx.f32_to_bf16(E)
    for c in g["cases"]:
        log(f"golden codebook case {c['name']}")
        lg = nx.f32_to_bf16(np.array(c["logits"], np.float32))[None]
        out, fr, seen, done, aligned = run_gpu_steps(
            H, [lg], np.array([c["frame"]], np.int32), np.array([c["eoc_seen"]], np.uint8),
            np.array([c["done"]], np.uint8), E_bits, V, g["bos"], g["eoc"], c["max_frames"])
        codes, emb = out[0]
        assert codes[0].tolist() == c["codes"], c["name"]
        assert int(fr[0]) == c["frame_out"] and int(done[0]) == c["done_out"], c["name"]
        assert seen[0].tolist() == c["eoc_seen_out"], c["name"]
        want = np.full_like(aligned, -1)
        for f, k, v in c["aligned_writes"]:
            want[0, f, k] = v
        np.testing.assert_array_equal(aligned, want, err_msg=c["name"])
        assert nx.bf16_to_f64(emb[0, :2]).tolist() == c["emb"], c["name"]


def _workload_vs_oracle(H, f32: bool):
    from gpu_util import log
    m = synth.QWEN3_4B
    B, K, V, steps, maxf = 64, m.n_codebooks, m.cb_vocab, 16, 40
    bos, eoc = m.bos_id, m.eoc_id
    E_bits = synth.codebook_embed(m)
    E = nx.bf16_to_f32(E_bits)
    st = synth.codebook_state(B, K)
    if f32:
        rng = np.random.default_rng(77)
        logits = [(rng.standard_normal((B, K, V)) * 2).astype(np.float32) for _ in range(steps)]
        for lg in logits:
            lg[rng.random((B, K)) < 0.05, eoc] = 9.0
    else:
        logits = [synth.codebook_logits(B, K, V, s, eoc) for s in range(steps)]
    log(f"codebook workload B={B} K={K} V={V} steps={steps} f32={f32}")
    gpu, fr, seen, done, aligned = run_gpu_steps(H, logits, st["frame"], st["eoc_seen"], st["done"], E_bits, V,
                                                 bos, eoc, maxf, f32=f32)
    o_frame, o_seen, o_done = st["frame"].copy(), st["eoc_seen"].copy(), st["done"].copy()
    o_aligned = np.full((B, maxf, K), -1, np.int32)
    for s in range(steps):
        lg = logits[s] if f32 else nx.bf16_to_f32(logits[s])
        codes, emb = oc.codebook_step(lg, o_frame, o_seen, o_done, bos, eoc, E, o_aligned, maxf)
        np.testing.assert_array_equal(gpu[s][0], codes, err_msg=f"codes step {s}")
        np.testing.assert_array_equal(gpu[s][1], emb, err_msg=f"emb step {s}")
    np.testing.assert_array_equal(fr, o_frame)
    np.testing.assert_array_equal(seen, o_seen)
    np.testing.assert_array_equal(done, o_done)
    np.testing.assert_array_equal(aligned, o_aligned)
    return o_done


def test_workload_bf16_logits_bit_exact(H):
    done = _workload_vs_oracle(H, f32=False)
    assert done.sum() >= 0


def test_workload_fp32_logits_bit_exact(H):
    _workload_vs_oracle(H, f32=True)


ODD_CASES = [
    # B, K, V, fp32 logits, tie-heavy: odd V puts rows at odd element offsets
    # (pairs straddle rows); K = 33 gives 8 lanes per codebook, V = 2000 takes
    # two load batches; integer-valued logits make most rows tie many times
    (3, 5, 77, False, False),
    (3, 5, 77, True, False),
    (2, 33, 301, False, True),
    (1, 8, 2000, True, False),
    (4, 8, 1026, False, True),
    (5, 3, 3, True, True),
]


@pytest.mark.parametrize("B,K,V,f32,ties", ODD_CASES, ids=[f"B{c[0]}_K{c[1]}_V{c[2]}_{'f32' if c[3] else 'bf16'}"
                                                           f"{'_ties' if c[4] else ''}" for c in ODD_CASES])
def test_odd_shapes_and_ties_bit_exact(H, B, K, V, f32, ties):
    from gpu_util import log
    rng = np.random.default_rng(1000 + B * 7 + K * 13 + V)
    D, steps, maxf = 16, 4, 8
    bos, eoc = V - 2, V - 1
    E_bits = nx.f32_to_bf16((rng.standard_normal((K * V, D)) * 0.5).astype(np.float32))
    E = nx.bf16_to_f32(E_bits)
    if ties:
        logits = [rng.integers(0, 4, (B, K, V)).astype(np.float32) for _ in range(steps)]
    else:
        logits = [(rng.standard_normal((B, K, V)) * 2).astype(np.float32) for _ in range(steps)]
    if not f32:
        logits = [nx.f32_to_bf16(lg) for lg in logits]
    frame = rng.integers(0, K + 2, B).astype(np.int32)
    seen = (rng.random((B, K)) < 0.2).astype(np.uint8)
    done = np.zeros(B, np.uint8)
    log(f"codebook odd case B={B} K={K} V={V} f32={f32} ties={ties}")
    gpu, fr, gseen, gdone, aligned = run_gpu_steps(H, logits, frame, seen, done, E_bits, V, bos, eoc, maxf,
                                                    f32=f32)
    o_frame, o_seen, o_done = frame.copy(), seen.copy(), done.copy()
    o_aligned = np.full((B, maxf, K), -1, np.int32)
    for s in range(steps):
        lg = logits[s] if f32 else nx.bf16_to_f32(logits[s])
        codes, emb = oc.codebook_step(lg, o_frame, o_seen, o_done, bos, eoc, E, o_aligned, maxf)
        np.testing.assert_array_equal(gpu[s][0], codes, err_msg=f"codes step {s}")
        np.testing.assert_array_equal(gpu[s][1], emb, err_msg=f"emb step {s}")
    np.testing.assert_array_equal(fr, o_frame)
    np.testing.assert_array_equal(gseen, o_seen)
    np.testing.assert_array_equal(gdone, o_done)
    np.testing.assert_array_equal(aligned, o_aligned)


def test_invalid_ids_refused(H):
    import torch
    d = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    z = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(H.HrError, match="HR_EINVAL"):
        H.hr_codebook_step(1, 2, 4, 3, 3, d, z, z, z, z, None, 0, d, 8, d)
