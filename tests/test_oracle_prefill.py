"""Pins of the float64 prefill oracle against closed forms, invariants and brute
force on tiny shapes.  Each test is chosen so that a plausible slip in the oracle
(dropped eps, wrong rotate-half sign or pairing, wrong GQA head map, transposed
weight, wrong gate/up order, causal off-by-one, wrong cache slot) fails it."""
import math
from dataclasses import dataclass

import numpy as np
import pytest

from oracle import prefill as op


@dataclass(frozen=True)
class Dims:
    hidden: int = 32
    n_q_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 8
    ffn: int = 24
    n_layers: int = 1
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6
    n_codebooks: int = 3
    cb_vocab: int = 5


def rand_layer(m, seed=0, scale=0.3):
    g = np.random.default_rng(seed)
    D, d = m.hidden, m.head_dim
    return {
        "in_norm": 1 + 0.1 * g.standard_normal(D),
        "post_norm": 1 + 0.1 * g.standard_normal(D),
        "q_norm": 1 + 0.1 * g.standard_normal(d),
        "k_norm": 1 + 0.1 * g.standard_normal(d),
        "w_qkv": scale * g.standard_normal(((m.n_q_heads + 2 * m.n_kv_heads) * d, D)),
        "w_o": scale * g.standard_normal((D, m.n_q_heads * d)),
        "w_gu": scale * g.standard_normal((2 * m.ffn, D)),
        "w_down": scale * g.standard_normal((D, m.ffn)),
    }


def batch_of(lens, cap, start=None, slots=None):
    lens = list(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return {"cu_seqlens": cu,
            "start_pos": np.zeros(len(lens), int) if start is None else np.array(start),
            "cache_slot": np.arange(len(lens)) if slots is None else np.array(slots),
            "capacity": cap}


# ----------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_matches_fsum_definition():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 37)) * 4
    w = 1 + 0.1 * g.standard_normal(37)
    got = op.rms_norm(x, w, 1e-6)
    for r in range(5):
        ms = math.fsum(float(v) * float(v) for v in x[r]) / 37
        inv = 1.0 / math.sqrt(ms + 1e-6)
        for j in range(37):
            assert got[r, j] == pytest.approx(x[r, j] * inv * w[j], rel=1e-14, abs=1e-15)


def test_rmsnorm_invariants():
    g = np.random.default_rng(4)
    x = g.standard_normal((4, 64))
    ones = np.ones(64)
    y = op.rms_norm(x, ones, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-5)
    np.testing.assert_allclose(op.rms_norm(7.5 * x, ones, 0.0), op.rms_norm(x, ones, 0.0), rtol=1e-13)
    assert np.all(op.rms_norm(np.zeros((2, 64)), ones, 1e-6) == 0)
    # eps matters for small rows: mean(x^2) = 1e-6 -> scale 1/sqrt(2e-6)
    t = np.full((1, 16), 1e-3)
    np.testing.assert_allclose(op.rms_norm(t, np.ones(16), 1e-6), 1e-3 / math.sqrt(2e-6), rtol=1e-12)


# ----------------------------------------------------------------------------- RoPE
def test_rope_is_complex_rotation_of_half_pairs():
    """Pair (m, m+d/2) as z = x_m + i x_{m+d/2}; RoPE multiplies z by e^{i p theta^(-2m/d)}."""
    g = np.random.default_rng(5)
    d, theta = 16, 1.0e6
    x = g.standard_normal((3, 2, d))
    pos = np.array([0, 7, 2047])
    y = op.apply_rope(x, pos, theta)
    for i, p in enumerate(pos):
        for hh in range(2):
            for mm in range(d // 2):
                z = complex(x[i, hh, mm], x[i, hh, mm + d // 2])
                w = z * complex(math.cos(p * theta ** (-2 * mm / d)), math.sin(p * theta ** (-2 * mm / d)))
                assert y[i, hh, mm] == pytest.approx(w.real, abs=1e-12)
                assert y[i, hh, mm + d // 2] == pytest.approx(w.imag, abs=1e-12)


def test_rope_invariants():
    g = np.random.default_rng(6)
    d = 128
    q = g.standard_normal((1, 1, d))
    k = g.standard_normal((1, 1, d))
    # p = 0 is the identity
    np.testing.assert_array_equal(op.apply_rope(q, np.array([0]), 1e6), q)
    # per-pair norms preserved
    y = op.apply_rope(q, np.array([1234]), 1e6)
    n0 = q[0, 0, :64] ** 2 + q[0, 0, 64:] ** 2
    n1 = y[0, 0, :64] ** 2 + y[0, 0, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # q.k depends only on the position offset
    def dot(pq, pk):
        return float(np.sum(op.apply_rope(q, np.array([pq]), 1e6) * op.apply_rope(k, np.array([pk]), 1e6)))
    assert dot(10, 3) == pytest.approx(dot(1010, 1003), abs=1e-9)
    assert dot(5, 5) == pytest.approx(float(np.sum(q * k)), abs=1e-12)
    # frequency of pair 0 is one radian per position
    e0 = np.zeros((1, 1, d)); e0[0, 0, 0] = 1.0
    r = op.apply_rope(e0, np.array([1]), 1e6)
    assert r[0, 0, 0] == pytest.approx(math.cos(1.0)) and r[0, 0, 64] == pytest.approx(math.sin(1.0))


# ----------------------------------------------------------------------------- attention
def brute_attention(q, K, V, visible):
    n, d = q.shape
    out = np.zeros((n, V.shape[1]))
    for i in range(n):
        s = [sum(q[i, t] * K[j, t] for t in range(d)) / math.sqrt(d) if visible[i, j] else None
             for j in range(K.shape[0])]
        mx = max(v for v in s if v is not None)
        e = [math.exp(v - mx) if v is not None else 0.0 for v in s]
        tot = math.fsum(e)
        for j in range(K.shape[0]):
            out[i] += e[j] / tot * V[j]
    return out


def test_attention_brute_force_and_invariants():
    g = np.random.default_rng(7)
    n, d = 5, 8
    q, K, V = g.standard_normal((n, d)), g.standard_normal((n, d)), g.standard_normal((n, d))
    causal = np.arange(n)[None, :] <= np.arange(n)[:, None]
    got = op.attention(q, K, V, causal)
    np.testing.assert_allclose(got, brute_attention(q, K, V, causal), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(got[0], V[0])                 # row 0 sees only key 0
    p = op.softmax(g.standard_normal((3, 9)))
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-15)
    # equal scores -> mean of the visible values
    z = op.attention(np.zeros((n, d)), K, V, causal)
    for i in range(n):
        np.testing.assert_allclose(z[i], V[:i + 1].mean(0), rtol=1e-13)
    # non-causal over s keys == causal row s-1
    full = op.attention(q[n - 1:], K, V, np.ones((1, n), bool))
    np.testing.assert_allclose(full[0], got[n - 1], rtol=1e-13)


# ----------------------------------------------------------------------------- layer
def run_layer(m, lw, lens, cap=16, start=None, slots=None, causal=True, used=None, h=None, caches=None):
    b = batch_of(lens, cap, start, slots)
    T = sum(lens)
    if h is None:
        h = np.random.default_rng(11).standard_normal((T, m.hidden))
    n_slots = (max(b["cache_slot"]) + 1) if len(lens) else 1
    kc, vc = caches if caches is not None else op.new_cache(m, n_slots, cap)
    out = op.prefill_layer(m, lw, b, h, kc, vc, causal, used)
    return out, kc, vc, h


def test_layer_zero_output_projections_leave_h_unchanged():
    m = Dims()
    lw = rand_layer(m)
    lw["w_o"][:] = 0
    lw["w_down"][:] = 0
    out, _, _, h = run_layer(m, lw, [6])
    np.testing.assert_array_equal(out, h)


def test_layer_single_token_attends_to_itself_and_splits_qkv_rows():
    """P = 1: attention returns v; with W_o selecting head outputs, h gains exactly
    the v rows of W_qkv (rows (Hq+Hkv)d ... ) applied to x, per the GQA map."""
    m = Dims()
    lw = rand_layer(m)
    lw["w_down"][:] = 0
    D, d, Hq, Hkv = m.hidden, m.head_dim, m.n_q_heads, m.n_kv_heads
    lw["w_o"] = np.eye(D, Hq * d)             # h[:, j] += o[:, j] for j < D
    out, kc, vc, h = run_layer(m, lw, [1])
    x = op.rms_norm(h, lw["in_norm"])
    v = x @ lw["w_qkv"][(Hq + Hkv) * d:].T    # [1, Hkv*d]
    o = np.concatenate([v[:, (hh // (Hq // Hkv)) * d:(hh // (Hq // Hkv) + 1) * d] for hh in range(Hq)], 1)
    np.testing.assert_allclose(out - h, o[:, :D] if o.shape[1] >= D else np.pad(o, ((0, 0), (0, D - o.shape[1]))),
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(vc[0], v.reshape(Hkv, d), rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv_heads():
    m = Dims()
    lw = rand_layer(m, seed=1)
    d, Hq, Hkv = m.head_dim, m.n_q_heads, m.n_kv_heads
    grp = Hq // Hkv
    wq = lw["w_qkv"][:Hq * d]
    wk = lw["w_qkv"][Hq * d:(Hq + Hkv) * d].reshape(Hkv, d, -1)
    wv = lw["w_qkv"][(Hq + Hkv) * d:].reshape(Hkv, d, -1)
    rep = lambda w: np.concatenate([w[hh // grp] for hh in range(Hq)], 0)
    mha = Dims(n_kv_heads=Hq)
    lw2 = dict(lw, w_qkv=np.concatenate([wq, rep(wk), rep(wv)], 0))
    a, *_ = run_layer(m, lw, [7])
    b, *_ = run_layer(mha, lw2, [7])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_swiglu_gate_then_up_closed_form():
    """W_o = 0; gate row j and up row j read x_0 with gains 0.7 / -1.3; W_down
    copies activation j into h_j: h_j += silu(0.7 x0) * (-1.3 x0)."""
    m = Dims()
    lw = rand_layer(m)
    lw["w_o"][:] = 0
    F, D = m.ffn, m.hidden
    lw["w_gu"][:] = 0
    lw["w_gu"][:F, 0] = 0.7
    lw["w_gu"][F:, 0] = -1.3
    lw["w_down"][:] = 0
    lw["w_down"][0, 0] = 1.0
    out, _, _, h = run_layer(m, lw, [3])
    x0 = op.rms_norm(h, lw["post_norm"])[:, 0]
    g = 0.7 * x0
    want = g / (1 + np.exp(-g)) * (-1.3 * x0)
    np.testing.assert_allclose(out[:, 0] - h[:, 0], want, rtol=1e-12)
    np.testing.assert_array_equal(out[:, 1:], h[:, 1:])


def test_packed_batch_equals_separate_sequences_and_slots():
    m = Dims()
    lw = rand_layer(m, seed=2)
    g = np.random.default_rng(12)
    lens = [5, 1, 8]
    h = g.standard_normal((sum(lens), m.hidden))
    out, kc, vc, _ = run_layer(m, lw, lens, cap=12, slots=[2, 0, 1], h=h)
    cu = np.concatenate([[0], np.cumsum(lens)])
    for s, slot in enumerate([2, 0, 1]):
        one, k1, v1, _ = run_layer(m, lw, [lens[s]], cap=12, h=h[cu[s]:cu[s + 1]])
        np.testing.assert_allclose(out[cu[s]:cu[s + 1]], one, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(kc[slot * 12: slot * 12 + lens[s]], k1[:lens[s]], rtol=1e-12, atol=1e-14)
        assert np.all(np.isnan(kc[slot * 12 + lens[s]: (slot + 1) * 12]))   # untouched slots


def test_prefill_in_two_calls_equals_one_call():
    """P tokens at once == P-1 tokens, then 1 token at start_pos P-1 reading the
    cache: pins causal visibility, RoPE positions and the cache slot formula."""
    m = Dims()
    lw = rand_layer(m, seed=3)
    h = np.random.default_rng(13).standard_normal((6, m.hidden))
    full, kf, vf, _ = run_layer(m, lw, [6], cap=10, slots=[1], h=h)
    caches = op.new_cache(m, 2, 10)
    a, *_ = run_layer(m, lw, [5], cap=10, slots=[1], h=h[:5], caches=caches)
    b, kc, vc, _ = run_layer(m, lw, [1], cap=10, start=[5], slots=[1], h=h[5:], caches=caches)
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kc[10:16], kf[10:16], rtol=1e-13, atol=1e-14)


def test_noncausal_pads_are_not_written_and_do_not_leak():
    m = Dims()
    lw = rand_layer(m, seed=4)
    h = np.random.default_rng(14).standard_normal((9, m.hidden))
    h[6:] = 0.0
    out, kc, _, _ = run_layer(m, lw, [9], cap=9, causal=False, used=[6], h=h)
    assert np.all(np.isnan(kc[6:9]))
    h2 = h.copy(); h2[6:] = 5.0                       # pad contents do not matter
    out2, *_ = run_layer(m, lw, [9], cap=9, causal=False, used=[6], h=h2)
    np.testing.assert_array_equal(out[:6], out2[:6])
    # every used query sees all six keys: equals the causal output of the last used row
    c, *_ = run_layer(m, lw, [6], cap=9, h=h[:6])
    np.testing.assert_allclose(out[5], c[5], rtol=1e-12)


def test_head_logits_layout():
    m = Dims()
    z = np.random.default_rng(15).standard_normal((2, m.hidden))
    w = np.zeros((m.n_codebooks * m.cb_vocab, m.hidden))
    w[1 * m.cb_vocab + 3, 4] = 2.0                      # codebook 1, id 3 reads z[:, 4]
    lg = op.head_logits(z, w, m.n_codebooks, m.cb_vocab)
    assert lg.shape == (2, m.n_codebooks, m.cb_vocab)
    np.testing.assert_array_equal(lg[:, 1, 3], 2.0 * z[:, 4])
    lg[:, 1, 3] = 0
    assert np.all(lg == 0)


def test_stack_composes_layers_and_final_norm():
    m = Dims(n_layers=2)
    lws = [rand_layer(m, seed=s) for s in (5, 6)]
    h0 = np.random.default_rng(16).standard_normal((4, m.hidden))
    wf = 1 + 0.1 * np.random.default_rng(17).standard_normal(m.hidden)
    b = batch_of([4], 8)
    caches = [op.new_cache(m, 1, 8) for _ in range(2)]
    hL, z, _ = op.prefill_stack(m, lambda l: lws[l], b, h0, caches, wf)
    h = h0
    for l in range(2):
        kc, vc = op.new_cache(m, 1, 8)
        h = op.prefill_layer(m, lws[l], b, h, kc, vc)
    np.testing.assert_array_equal(hL, h)
    np.testing.assert_array_equal(z, op.rms_norm(h, wf))


# ----------------------------------------------------------------------------- per-head q/k norm
def _scalar_qk_attention(m, lw, h, start):
    """Independent scalar evaluation of steps 1-6 of the layer for one causal
    sequence at positions start, start+1, ... ("Stabilize Higgs Audio
    termination and prefill", Summary: q/k norm + RoPE, then attention).
    Per head, over its d values: RMS with its own weight (q_norm for query
    heads, k_norm for key heads), THEN the rotation, written as the complex
    product (x_m + i x_{m+d/2}) * exp(i p theta^(-2m/d)).  Returns the rotated
    keys [T][Hkv][d] and the attention outputs [T][Hq][d] as Python floats."""
    import cmath
    D, Hq, Hkv, d = m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim
    eps, theta, half = m.rms_eps, m.rope_theta, m.head_dim // 2
    T = h.shape[0]
    W = [[float(v) for v in row] for row in lw["w_qkv"]]

    def rms(vals, w):
        ms = math.fsum(v * v for v in vals) / len(vals)
        inv = 1.0 / math.sqrt(ms + eps)
        return [v * inv * float(wj) for v, wj in zip(vals, w)]

    def rotate(vals, p):
        out = [0.0] * d
        for mm in range(half):
            z = complex(vals[mm], vals[mm + half]) * cmath.exp(1j * p * theta ** (-2.0 * mm / d))
            out[mm], out[mm + half] = z.real, z.imag
        return out

    qs, ks, vs = [], [], []
    for t in range(T):
        x = rms([float(v) for v in h[t]], lw["in_norm"])
        row = [math.fsum(x[j] * W[n][j] for j in range(D)) for n in range(len(W))]
        p = start + t
        qs.append([rotate(rms(row[hh * d:(hh + 1) * d], lw["q_norm"]), p) for hh in range(Hq)])
        kb = Hq * d
        ks.append([rotate(rms(row[kb + g * d:kb + (g + 1) * d], lw["k_norm"]), p) for g in range(Hkv)])
        vb = (Hq + Hkv) * d
        vs.append([row[vb + g * d:vb + (g + 1) * d] for g in range(Hkv)])
    outs = []
    for i in range(T):
        per_head = []
        for hh in range(Hq):
            g = hh // (Hq // Hkv)
            sc = [math.fsum(a * b for a, b in zip(qs[i][hh], ks[j][g])) / math.sqrt(d) for j in range(i + 1)]
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            tot = math.fsum(e)
            per_head.append([math.fsum(e[j] * vs[j][g][c] for j in range(i + 1)) / tot for c in range(d)])
        outs.append(per_head)
    return ks, outs


def test_qk_norm_per_head_with_own_weight_before_rope():
    """Cache keys and attention outputs of a 5-token prompt against the scalar
    evaluation above, with q_norm and k_norm far apart (a swapped weight, a
    norm across heads, a norm after the rotation or a dropped norm each move
    the result by orders of magnitude more than the tolerance)."""
    m = Dims(rope_theta=10.0)
    lw = rand_layer(m, seed=21, scale=0.4)
    g = np.random.default_rng(22)
    lw["q_norm"] = 1.0 + 0.6 * g.standard_normal(m.head_dim)
    lw["k_norm"] = 0.5 + 0.4 * g.standard_normal(m.head_dim)
    T = 5
    h = g.standard_normal((T, m.hidden))
    kc, vc = op.new_cache(m, 1, 16)
    taps = {}
    op.prefill_layer(m, lw, batch_of([T], 16), h, kc, vc, True, taps=taps)
    ks, outs = _scalar_qk_attention(m, lw, h, 0)
    np.testing.assert_allclose(kc[:T], np.array(ks), rtol=1e-11, atol=1e-12)
    o = taps["o"].reshape(T, m.n_q_heads, m.head_dim)
    np.testing.assert_allclose(o, np.array(outs), rtol=1e-10, atol=1e-11)


def test_qk_norm_removes_the_scale_of_each_head_alone():
    """Scaling the W_qkv rows of ONE query head (or one key head) by c > 0
    leaves the layer output unchanged when the RMSNorm runs per head (eps 0);
    a norm over all heads at once would let that head's scale move the
    others."""
    m = Dims(rms_eps=0.0, rope_theta=100.0)
    lw = rand_layer(m, seed=23)
    d, Hq = m.head_dim, m.n_q_heads
    ref, *_ = run_layer(m, lw, [6])
    for rows in (slice(1 * d, 2 * d), slice((Hq + 1) * d, (Hq + 2) * d)):   # q head 1, k head 1
        lw2 = {k: v.copy() for k, v in lw.items()}
        lw2["w_qkv"][rows] *= 3.7
        got, *_ = run_layer(m, lw2, [6])
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)
    # the v rows carry no norm: the same scale on a value head changes the output
    lw3 = {k: v.copy() for k, v in lw.items()}
    lw3["w_qkv"][(Hq + 2) * d:(Hq + 3) * d] *= 3.7
    got, *_ = run_layer(m, lw3, [6])
    assert np.max(np.abs(got - ref)) > 1e-3


def test_qk_norm_weights_are_not_interchangeable():
    m = Dims(rope_theta=10.0)
    lw = rand_layer(m, seed=24)
    lw["q_norm"] = np.linspace(0.3, 1.9, m.head_dim)
    lw["k_norm"] = np.linspace(1.7, 0.2, m.head_dim)
    ref, kc_ref, *_ = run_layer(m, lw, [5])
    lw2 = dict(lw, q_norm=lw["k_norm"], k_norm=lw["q_norm"])
    got, kc_got, *_ = run_layer(m, lw2, [5])
    assert np.max(np.abs(got - ref)) > 1e-3
    assert np.max(np.abs(kc_got[:5] - kc_ref[:5])) > 1e-2
