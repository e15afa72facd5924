"""Pins of the MXFP4 oracle (no GPU).

* E2M1 against the element table of the OCP MX specification (all 16 codes),
  hand-worked midpoints (ties to the even code) and saturation.
* Block scales against hand-worked blocks: the shared exponent floor(log2 amax)
  - 2, its clamp, the zero block, exact round trips of representable blocks and
  the clipping the rule implies.
* The blocked product against brute force over decoded elements.
* AWQ: the closed form on hand values, its clamp, and the invariance that makes
  it safe: without quantisation the pre-scaled layer equals the plain layer
  (a wrong fold direction or axis fails this).
"""
import numpy as np
import pytest

import synth
from oracle import mxfp4 as mx
from oracle import prefill as op

# OCP MX v1.0, FP4 (E2M1) element values: codes 0..7 positive, 8..15 negative
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_decode_table():
    got = mx.e2m1_decode(np.arange(16))
    assert got.tolist() == SPEC_E2M1
    assert np.signbit(got[8])


def test_e2m1_encode_round_trip_midpoints_saturation():
    vals = np.array(SPEC_E2M1)
    assert mx.e2m1_encode(vals).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, 0, 9, 10, 11, 12, 13, 14, 15]
    # midpoints between neighbours go to the even code (mantissa bit 0)
    mids = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in mids.items():
        assert int(mx.e2m1_encode(x)) == c, x
        assert int(mx.e2m1_encode(-x)) == (c | 8 if c else 0), -x
    assert int(mx.e2m1_encode(0.2500001)) == 1 and int(mx.e2m1_encode(0.7499999)) == 1
    assert int(mx.e2m1_encode(5.0000001)) == 7 and int(mx.e2m1_encode(4.9999999)) == 6
    assert mx.e2m1_encode([6.5, 7.0, 1e9, -1e9]).tolist() == [7, 7, 7, 15]


def test_block_scale_exponent_cases():
    cases = {6.0: 0, 1.0: -2, 7.99: 0, 8.0: 1, 0.5: -3, 3.0: -1, 2.0 ** -130: -127, 0.0: -127,
             2.0 ** 130: 127}
    for a, e in cases.items():
        assert int(mx.block_scale_exp(a)) == e, a


def test_block_quantise_round_trip_and_clipping():
    rng = np.random.default_rng(0)
    # a representable block: E2M1 values times 2^e, with a 6 or -6 present
    for e in (-5, 0, 3):
        codes = rng.integers(0, 16, 32)
        codes[rng.integers(0, 32)] = 7
        v = mx.e2m1_decode(codes) * 2.0 ** e
        q, s = mx.quantize_blocks(v[None])
        assert int(s[0, 0]) == 127 + e
        np.testing.assert_array_equal(mx.dequantize_blocks(q, s)[0], v)
    # amax 7: e = floor(log2 7) - 2 = 0, so 7 clips to 6 and 1.25 rounds to 1
    q, s = mx.quantize_blocks(np.array([[7.0, 1.25] + [0.0] * 30]))
    assert int(s[0, 0]) == 127 and mx.dequantize_blocks(q, s)[0, :2].tolist() == [6.0, 1.0]
    q, s = mx.quantize_blocks(np.zeros((1, 64)))
    assert s.tolist() == [[0, 0]] and not q.any()


def test_pack_nibble_order():
    c = np.arange(16, dtype=np.uint8)
    p = mx.pack_codes(c)
    assert p.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    np.testing.assert_array_equal(mx.unpack_codes(p), c)


def test_blocked_product_brute_force():
    rng = np.random.default_rng(1)
    M, N, K = 3, 4, 96
    a = rng.normal(0, 1, (M, K)) * np.exp(rng.normal(0, 2, (M, 1)))
    b = rng.normal(0, 1, (N, K))
    ac, as_ = mx.quantize_blocks(a)
    bc, bs = mx.quantize_blocks(b)
    y = mx.mx_matmul(ac, as_, bc, bs)
    for i in range(M):
        for j in range(N):
            acc = 0.0
            for k in range(K):
                xa = SPEC_E2M1[int(ac[i, k])] * 2.0 ** (int(as_[i, k // 32]) - 127)
                xb = SPEC_E2M1[int(bc[j, k])] * 2.0 ** (int(bs[j, k // 32]) - 127)
                acc += xa * xb
            assert y[i, j] == pytest.approx(acc, rel=1e-12, abs=1e-300)


def test_awq_scale_closed_form_and_clamp():
    s = mx.awq_scale(np.array([4.0, 1.0, 1.0, 1.0, 1.0]), 0.8)
    mean = 8.0 / 5.0
    assert s[0] == pytest.approx((4.0 / mean) ** 0.8) and s[1] == pytest.approx((1.0 / mean) ** 0.8)
    assert mx.awq_scale(np.ones(7)).tolist() == [1.0] * 7
    a = np.array([100.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1e-9, 20.0])     # mean 14
    s = mx.awq_scale(a)
    assert s[0] == 4.0 and s[7] == 0.25 and s[1] == 0.25            # (7.1)^0.8 > 4, (0.07)^0.8 < 0.25
    assert s[8] == pytest.approx((20.0 / (126.0 + 1e-6) * 9) ** 0.8)


def test_awq_fold_preserves_the_layer():
    """With exact products, O / gate-up / down with the pre-scale folded as the
    band folds it equal the plain layer."""
    m = synth.TINY
    lw = op.widen_layer(synth.layer_tensors(m, 0))
    rng = np.random.default_rng(2)
    awq = {"o": rng.uniform(0.25, 4, m.n_q_heads * m.head_dim), "gu": rng.uniform(0.25, 4, m.hidden),
           "dn": rng.uniform(0.25, 4, m.ffn)}
    F = m.ffn
    w2 = dict(lw)
    w2["w_o"] = lw["w_o"] * awq["o"][None, :]
    w2["w_gu"] = lw["w_gu"] * awq["gu"][None, :]
    w2["w_gu"][F:] = w2["w_gu"][F:] / awq["dn"][:, None]
    w2["w_down"] = lw["w_down"] * awq["dn"][None, :]

    def lin(site, x, w):
        if site == "o":
            x = x / awq["o"][None, :]
        if site == "gu":
            x = x / awq["gu"][None, :]
        return x @ w.T
    T = 6
    h = rng.normal(0, 1, (T, m.hidden))
    batch = {"cu_seqlens": np.array([0, T]), "start_pos": np.array([0]), "cache_slot": np.array([0]),
             "capacity": 8}
    c1 = op.new_cache(m, 1, 8, 0.0)
    c2 = op.new_cache(m, 1, 8, 0.0)
    ref = op.prefill_layer(m, lw, batch, h, *c1)
    got = op.prefill_layer(m, w2, batch, h, *c2, linear=lin)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_mx_layer_close_to_plain_and_packing_consistent():
    """The band's layer on the tiny model: packing = quantize_blocks of the
    binary32 pre-scaled weight, and the quantised layer stays near the plain
    one (4-bit operands: a loose bound, the GPU is held to the quantised layer)."""
    m = synth.TINY
    lw = op.widen_layer(synth.layer_tensors(m, 0))
    h0 = op.widen_layer({"x": synth.embed_rows(m, synth.calibration_ids(m))})["x"]
    awq = mx.calibrate_awq(m, lw, h0)
    for site, n in (("o", m.n_q_heads * m.head_dim), ("gu", m.hidden), ("dn", m.ffn)):
        assert awq[site].shape == (n,) and np.all((awq[site] >= 0.25) & (awq[site] <= 4.0))
    lw32 = {k: v.astype(np.float32) for k, v in lw.items()}
    pk = mx.pack_layer(lw32, awq)
    c, s = pk["packed"]["dn"]
    c2, s2 = mx.quantize_blocks((lw32["w_down"] * pk["col"]["dn"][None, :]).astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(c, c2)
    np.testing.assert_array_equal(s, s2)
    T = 6
    h = op.widen_layer({"x": synth.embed_rows(m, synth.prompt_ids(m, T))})["x"]
    batch = {"cu_seqlens": np.array([0, T]), "start_pos": np.array([0]), "cache_slot": np.array([0]),
             "capacity": 8}
    ref = op.prefill_layer(m, lw, batch, h, *op.new_cache(m, 1, 8, 0.0))
    got = mx.mx_layer(m, lw, pk, batch, h, *op.new_cache(m, 1, 8, 0.0))
    d_ref, d_got = (ref - h).ravel(), (got - h).ravel()
    cos = d_ref @ d_got / np.linalg.norm(d_ref) / np.linalg.norm(d_got)
    assert cos > 0.9, cos
