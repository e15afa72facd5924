"""Pins of the FP8 oracle: weight packing against torch's E4M3 cast, calibration
statistic and refusal, and the fake-quant product on exactly representable data."""
import numpy as np
import pytest
import torch

from oracle import fp8 as of
from oracle import numerics as nx
from oracle import prefill as op
from test_oracle_prefill import Dims, rand_layer


def test_weight_packing_per_output_channel():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((40, 96)) * 0.02).astype(np.float32)
    s, codes = of.weight_scales_e4m3(w)
    assert s.dtype == np.float32 and s.shape == (40,)
    np.testing.assert_array_equal(s, (np.abs(w).max(1) / np.float32(448.0)).astype(np.float32))
    q32 = (w / s[:, None]).astype(np.float32)
    want = torch.from_numpy(q32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(nx.e4m3_decode(codes), nx.e4m3_decode(want))
    # each row's largest magnitude lands on +-448 exactly
    row_max = np.abs(nx.e4m3_decode(codes)).max(1)
    np.testing.assert_array_equal(row_max, 448.0)
    # reconstruction within half an E4M3 step (relative 2^-4) of the original
    rec = nx.e4m3_decode(codes) * s[:, None]
    big = np.abs(w) > 2.0 ** -6 * s[:, None]            # normal range of E4M3
    assert np.all(np.abs(rec - w)[big] <= np.abs(w)[big] * 2.0 ** -4 * 1.0001)


def test_calibration_takes_raw_peak_at_the_four_sites():
    m = Dims()
    lw = rand_layer(m, seed=8)
    h0 = np.random.default_rng(32).standard_normal((7, m.hidden))
    sc = of.calibrate(m, lw, h0)
    taps = {}
    kc, vc = op.new_cache(m, 1, 7, 0.0)
    op.prefill_layer(m, lw, {"cu_seqlens": [0, 7], "start_pos": [0], "cache_slot": [0], "capacity": 7},
                     h0, kc, vc, False, [7], taps=taps)
    for site in of.SITES:
        assert sc[site] == pytest.approx(np.abs(taps[site]).max() / 448.0, rel=1e-15)
    # the gu input is the post-attention norm output, the dn input is silu(g)*u
    assert taps["qkv"].shape == (7, m.hidden) and taps["dn"].shape == (7, m.ffn)


def test_calibration_refuses_a_dead_site():
    m = Dims()
    lw = rand_layer(m, seed=9)
    lw["w_qkv"][(m.n_q_heads + m.n_kv_heads) * m.head_dim:] = 0.0      # v = 0 -> o = 0
    with pytest.raises(ValueError, match="dead quantizer site o"):
        of.calibrate(m, lw, np.random.default_rng(33).standard_normal((5, m.hidden)))


def test_fake_quant_is_exact_on_representable_operands():
    rng = np.random.default_rng(34)
    vals = nx.E4M3_VALUES[np.r_[1:127, 129:255]]
    a = 0.25
    s_w = np.full(12, 0.5, np.float32)
    x = rng.choice(vals, (5, 20)) * a
    w8 = rng.choice(vals, (12, 20))
    codes = nx.e4m3_encode(w8)
    lin = of.fake_quant_linear({"qkv": a}, {"qkv": (s_w, codes)})
    got = lin("qkv", x, None)
    np.testing.assert_allclose(got, x @ (w8 * 0.5).T, rtol=1e-14, atol=1e-14)


def test_fp8_layer_tracks_the_unquantised_layer():
    """With calibrated scales the fake-quant layer stays close to the exact one
    (the relative error budget of E4M3 is a few percent per element)."""
    m = Dims(hidden=64, ffn=96, head_dim=16)
    lw = rand_layer(m, seed=10, scale=0.1)
    h = np.random.default_rng(35).standard_normal((12, m.hidden))
    sc = of.calibrate(m, lw, h)
    packed = of.pack_layer({k: v.astype(np.float32) for k, v in lw.items()})
    b = {"cu_seqlens": [0, 12], "start_pos": [0], "cache_slot": [0], "capacity": 12}
    k1, v1 = op.new_cache(m, 1, 12)
    exact = op.prefill_layer(m, lw, b, h, k1, v1, False, [12])
    k2, v2 = op.new_cache(m, 1, 12)
    fq = of.fp8_layer(m, lw, sc, packed, b, h, k2, v2, False, [12])
    cos = np.sum(exact * fq) / np.linalg.norm(exact) / np.linalg.norm(fq)
    assert cos > 0.999
    assert not np.allclose(exact, fq, rtol=1e-6)          # it really quantised
