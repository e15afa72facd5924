"""The seeded input generators: determinism, blockwise consistency, distributions."""
import numpy as np

import synth


def test_blockwise_rows_equal_full_tensor_rows(monkeypatch):
    monkeypatch.setattr(synth, "BLOCK", 1000)           # force many blocks
    full = synth.normal_bf16((37, 77), (9, 1, 2), 0.02)
    rows = np.array([0, 36, 12, 13, 12])
    np.testing.assert_array_equal(synth.normal_bf16_rows((37, 77), rows, (9, 1, 2), 0.02), full[rows])
    again = synth.normal_bf16((37, 77), (9, 1, 2), 0.02, threads=1)
    np.testing.assert_array_equal(full, again)


def test_distributions_and_rounding():
    w = synth.bf16_bits_to_f32(synth.normal_bf16((512, 512), (9, 0, 5), 0.02))
    assert abs(float(w.mean())) < 2e-4 and abs(float(w.std()) - 0.02) < 2e-4
    n = synth.bf16_bits_to_f32(synth.normal_bf16((4096,), (9, 0, 1), 0.1, 1.0))
    assert abs(float(n.mean()) - 1.0) < 0.01 and abs(float(n.std()) - 0.1) < 0.01
    x = np.float32([1.0, 1.00390625, 1.01171875, 1.005859375])  # exact, tie down, tie up, nearest
    assert synth.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81]


def test_ids_lengths_and_logits():
    m = synth.TINY
    ids = synth.prompt_ids(m, 1000)
    assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < m.vocab
    np.testing.assert_array_equal(ids, synth.prompt_ids(m, 1000))
    lens = synth.varlen_lengths(32, 6, 256)
    assert lens.min() >= 6 and lens.max() <= 256 and lens.size == 32
    B, K, V = 64, 8, 1026
    lg = synth.codebook_logits(B, K, V, step=0, eoc_id=V - 1)
    vals = synth.bf16_bits_to_f32(lg)
    top = vals.argmax(-1)
    forced = top == V - 1
    assert 0.01 < forced.mean() < 0.12
    srt = np.sort(vals, -1)
    assert np.all(srt[..., -1][forced] > srt[..., -2][forced])      # strictly top-1
    st = synth.codebook_state(B, K)
    assert st["frame"].min() >= 0 and st["frame"].max() < 16


def test_workloads_named_with_sizes():
    w = synth.workloads()
    assert w["stack36_d2560_p512"].model.n_layers == 36
    v = w["varlen32_stack36_d2560"]
    assert len(v.prompt_lens) == 32 and v.capacity == 256
    assert w["fp8_layer_d2560_p512_pad544"].padded_rows == 544
