"""Each prefill step on the GPU against the float64 oracle, on seeded inputs,
through the C ABI (include/hr_ops.h).  Sizes span several tiles with ragged
tails; caches and outputs are NaN-poisoned to catch unwritten or stray writes.
Activation formats of the bf16-weight band: norm outputs, q, the attention
output and the SwiGLU product fp16; merged QKV rows fp32; caches bf16."""
import numpy as np
import pytest

import synth
from oracle import numerics as nx
from oracle import prefill as op
from oracle import fp8 as of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def seeded_bf16(shape, key, std=1.0, mean=0.0):
    return synth.normal_bf16(shape, (90,) + tuple(key), std, mean)


# ----------------------------------------------------------------------------- A0 / A1 / A6 / A9
@pytest.mark.parametrize("T,D", [(13, 2560), (300, 256), (1, 2560)])
def test_embed_rmsnorm_and_rmsnorm(H, T, D):
    import torch
    from gpu_util import assert_f16_close, dev, dev_bf16, f64_of, log
    log(f"embed_rmsnorm T={T} D={D}")
    vocab = 4096
    E = seeded_bf16((vocab, D), (1, D), 0.02)
    w = seeded_bf16((D,), (2, D), 0.1, 1.0)
    ids = np.random.default_rng(T).integers(0, vocab, T).astype(np.int32)
    h = torch.empty((T, D), dtype=torch.float32, device="cuda")
    x = torch.empty((T, D), dtype=torch.float16, device="cuda")
    H.hr_embed_rmsnorm(dev(ids), dev_bf16(E), vocab, None, T, D, dev_bf16(w), 1e-6, h, x)
    torch.cuda.synchronize()
    rows = nx.bf16_to_f64(E[ids])
    np.testing.assert_array_equal(h.cpu().numpy().astype(np.float64), rows)     # exact widening
    ref = op.rms_norm(rows, nx.bf16_to_f64(w), 1e-6)
    assert_f16_close(f64_of(x), ref, what="embed_rmsnorm x")
    # plain RMSNorm of an fp32 residual with larger spread
    hr = (np.random.default_rng(5).standard_normal((T, D)) * 7).astype(np.float32)
    x2 = torch.empty((T, D), dtype=torch.float16, device="cuda")
    H.hr_rmsnorm(dev(hr), T, D, dev_bf16(w), 1e-6, x2)
    torch.cuda.synchronize()
    assert_f16_close(f64_of(x2), op.rms_norm(hr.astype(np.float64), nx.bf16_to_f64(w), 1e-6),
                     what="rmsnorm x")


def test_rmsnorm_fp8_output(H):
    import torch
    from gpu_util import dev, dev_bf16
    T, D, a = 40, 2560, 0.03
    w = seeded_bf16((D,), (3,), 0.1, 1.0)
    hr = (np.random.default_rng(6).standard_normal((T, D)) * 3).astype(np.float32)
    x8 = torch.empty((T, D), dtype=torch.uint8, device="cuda")
    H.hr_rmsnorm(dev(hr), T, D, dev_bf16(w), 1e-6, x8, H.HR_FP8_E4M3, a)
    torch.cuda.synchronize()
    got = nx.e4m3_decode(x8.cpu().numpy())
    ref = op.rms_norm(hr.astype(np.float64), nx.bf16_to_f64(w), 1e-6) / a
    want = nx.e4m3_round(ref)
    # the fp32 and float64 quotients round to the same code except within
    # rounding distance of a midpoint: allow one code step on a tiny fraction
    diff = got != want
    assert diff.mean() < 1e-3
    step = np.abs(want) * 2.0 ** -3 + 2.0 ** -9
    assert np.all(np.abs(got - want)[diff] <= step[diff])


# ----------------------------------------------------------------------------- A2 / A5 / A7 / A8
def _linear_case(H, M, N, K, epi, fp8=False, seed=0):
    import torch
    from gpu_util import dev, dev_bf16, dev_f16, dev_u8, f64_of, log, seeded_f16
    log(f"linear M={M} N={N} K={K} epi={epi} fp8={fp8}")
    rng = np.random.default_rng(seed)
    if fp8:
        codes_x = rng.integers(0, 256, (M, K)).astype(np.uint8)
        codes_w = rng.integers(0, 256, (N, K)).astype(np.uint8)
        for c in (codes_x, codes_w):                        # no NaN codes
            c[(c & 0x7F) == 0x7F] = 0x3C
        xs, ws = 0.05, (rng.random(N) * 0.01 + 0.001).astype(np.float32)
        xv = nx.e4m3_decode(codes_x) * xs
        wv = nx.e4m3_decode(codes_w) * ws[:, None].astype(np.float64)
        dx, dw, dws = dev_u8(codes_x), dev_u8(codes_w), dev(ws)
        wtype = H.HR_FP8_E4M3
    else:
        # fp16 activations (seeded normals rounded to fp16) times bf16 weights
        xh = seeded_f16((M, K), 1000 * M + K + seed, 1.0)
        wb = seeded_bf16((N, K), (11, N, K, seed), 0.02)
        xv, wv = xh.astype(np.float64), nx.bf16_to_f64(wb)
        dx, dw, dws, xs = dev_f16(xh), dev_bf16(wb), None, 1.0
        wtype = H.HR_BF16
    ref = xv @ wv.T
    if epi == H.HR_EPI_F32:
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        H.hr_linear(dx, dw, dws, xs, wtype, M, N, K, epi, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        if fp8:
            absdot = np.abs(xv) @ np.abs(wv).T
            assert np.all(err <= 2.0 ** -11 * absdot + 1e-12), float(np.max(err / absdot))
        else:
            # exact products, fp32 accumulation
            scale = np.sqrt(np.sum(xv ** 2, 1))[:, None] * np.sqrt(np.sum(wv ** 2, 1))[None, :]
            assert np.all(err <= 1e-5 * scale), float(err.max())
    elif epi == H.HR_EPI_RESIDUAL:
        h0 = np.random.default_rng(seed + 1).standard_normal((M, N)).astype(np.float32)
        h = dev(h0)
        H.hr_linear(dx, dw, dws, xs, wtype, M, N, K, epi, h, ws=H.linear_ws(wtype, M, N, K, epi))
        torch.cuda.synchronize()
        got = h.cpu().numpy().astype(np.float64)
        want = h0 + ref
        if fp8:
            # the E4M3 MFMA sums its products with less than fp32 precision:
            # bound the error by a fraction of sum_k |x_k w_k|
            absdot = np.abs(xv) @ np.abs(wv).T
            ratio = float(np.max(np.abs(got - want) / absdot))
            log(f"fp8 residual max |err| / sum|x w| = {ratio:.3g}")
            assert ratio <= 2.0 ** -11, ratio
        else:
            scale = np.sqrt(np.sum(xv ** 2, 1))[:, None] * np.sqrt(np.sum(wv ** 2, 1))[None, :]
            assert np.all(np.abs(got - want) <= 1e-5 * scale + 2e-6 * np.abs(want)), float(np.abs(got - want).max())
    else:
        F = N // 2
        out_scale = 0.02
        if fp8:
            out = torch.empty((M, F), dtype=torch.uint8, device="cuda")
        else:
            out = torch.empty((M, F), dtype=torch.float16, device="cuda")
        H.hr_linear(dx, dw, dws, xs, wtype, M, N, K, epi, out, out_scale if fp8 else 0.0)
        torch.cuda.synchronize()
        act = op.silu(ref[:, :F]) * ref[:, F:]
        if fp8:
            got = nx.e4m3_decode(out.cpu().numpy()) * out_scale
            want = nx.e4m3_round(act / out_scale) * out_scale
            # the pre-quantisation value carries the E4M3 MFMA's accumulation
            # error (<= 2^-11 sum|x w| per product, measured on the residual
            # case); propagate it through silu(g) u and add half an E4M3 step
            absdot = np.abs(xv) @ np.abs(wv).T
            g, u = ref[:, :F], ref[:, F:]
            sig = 1 / (1 + np.exp(-g))
            dsilu = sig * (1 + g * (1 - sig))
            pre_err = 2.0 ** -11 * (np.abs(dsilu * u) * absdot[:, :F] + np.abs(op.silu(g)) * absdot[:, F:])
            # E4M3 saturates at 448 x out_scale
            sat = np.clip(act, -448.0 * out_scale, 448.0 * out_scale)
            bound = pre_err + np.abs(sat) * 2.0 ** -4 + 2.0 ** -10 * out_scale + 1e-12
            assert np.all(np.abs(got - sat) <= bound * 1.01), float(np.max(np.abs(got - sat) / bound))
            log(f"fp8 SwiGLU codes differing from the float64 quantisation: {float((got != want).mean()):.4f}")
        else:
            got = f64_of(out)
            gs = np.sqrt(np.sum(xv ** 2, 1))[:, None] * np.sqrt(np.sum(wv[:F] ** 2, 1) + np.sum(wv[F:] ** 2, 1))[None, :]
            assert np.all(np.abs(got - act) <= 2.0 ** -10 * np.abs(act) + 1e-4 * gs), float(np.abs(got - act).max())


@pytest.mark.parametrize("M", [1, 13, 16])
def test_linear_skinny_bf16(H, M):
    _linear_case(H, M, 6144, 2560, H.HR_EPI_F32, seed=M)
    _linear_case(H, M, 2560, 4096, H.HR_EPI_RESIDUAL, seed=M)
    _linear_case(H, M, 2 * 768, 256, H.HR_EPI_SWIGLU, seed=M)


@pytest.mark.parametrize("M", [17, 40, 64, 65, 200, 544])
def test_linear_tiled_bf16(H, M):
    _linear_case(H, M, 512, 2560, H.HR_EPI_F32, seed=M)
    _linear_case(H, M, 256, 768, H.HR_EPI_RESIDUAL, seed=M)
    _linear_case(H, M, 2560, 1024, H.HR_EPI_RESIDUAL, seed=M + 1)
    _linear_case(H, M, 2 * 768, 256, H.HR_EPI_SWIGLU, seed=M)


# the down projection's shapes (N 2560, K 9728) at every row range whose tile
# the dispatch picks differently: 17-64 rows, 65-128 (the 128-row prefill),
# 129-384, 385-576 (the 512-row prefill, 128 x 128 tiles split 3), 577-1024
# (256 x 128 split 6) and above 1024
@pytest.mark.parametrize("M", [17, 64, 65, 128, 129, 512, 600, 1100])
def test_linear_down_shapes(H, M):
    _linear_case(H, M, 2560, 9728, H.HR_EPI_RESIDUAL, seed=M + 7)


# 13 rows: skinny; 200: tiled; 512: the 385-576-row e4m3 tiles (192 x 256
# SwiGLU, 128 x 128 residual split 2)
@pytest.mark.parametrize("M", [13, 200, 512])
def test_linear_fp8(H, M):
    _linear_case(H, M, 512, 1024, H.HR_EPI_F32, fp8=True, seed=M)
    _linear_case(H, M, 256, 512, H.HR_EPI_RESIDUAL, fp8=True, seed=M)
    _linear_case(H, M, 2 * 256, 512, H.HR_EPI_SWIGLU, fp8=True, seed=M)


def test_linear_rejects_bad_shapes(H):
    import torch
    x = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.HrError, match="HR_EUNSUPPORTED"):
        H.hr_linear(x, x, None, 1.0, H.HR_BF16, 1, 16, 48, H.HR_EPI_F32, x)


# ----------------------------------------------------------------------------- A6 / A9 fused
# D sets the chunks per thread (2560: 2, 256: 1, 6144: 3, 8192: 4); ks above 4
# takes several batches of partial loads
@pytest.mark.parametrize("T,D,ks,fmt", [(13, 2560, 5, "f16"), (512, 2560, 6, "f16"), (300, 256, 1, "e4m3"),
                                        (7, 2560, 0, "f16"), (40, 2560, 3, "none"), (9, 8192, 6, "f16"),
                                        (5, 6144, 3, "e4m3"), (3, 4096, 9, "none")])
def test_residual_rmsnorm(H, T, D, ks, fmt):
    """h += p0 + ... + p_{ks-1} (split order), then RMS(h) * w in fp16 / e4m3
    (or nothing), against float64; run twice on the same inputs the bits must
    repeat; hr_linear's residual path (the same order) plus hr_rmsnorm give
    the same bits as the fused call."""
    import torch
    from gpu_util import assert_f16_close, dev, dev_bf16, f64_of, log
    log(f"residual_rmsnorm T={T} D={D} ks={ks} {fmt}")
    rng = np.random.default_rng(T * 31 + ks)
    h0 = (rng.standard_normal((T, D)) * 20).astype(np.float32)
    parts = (rng.standard_normal((max(ks, 1), T, D)) * 2).astype(np.float32)
    w = seeded_bf16((D,), (4, D), 0.1, 1.0)
    a = 0.05
    xtype = {"f16": H.HR_F16, "e4m3": H.HR_FP8_E4M3, "none": H.HR_F16}[fmt]
    outs = []
    for rep in range(2):
        h = dev(h0.copy())
        x = None if fmt == "none" else torch.empty((T, D), dtype=torch.uint8 if fmt == "e4m3" else torch.float16,
                                                   device="cuda")
        H.hr_residual_rmsnorm(h, dev(parts), ks, T, D, dev_bf16(w), 1e-6, x, xtype, a)
        torch.cuda.synchronize()
        outs.append((h.cpu().numpy(), None if x is None else x.cpu().numpy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    if fmt != "none":
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
    # the sum in split order, in fp32 (the contract), then added to h
    s = parts[0].copy() if ks > 0 else np.zeros((T, D), np.float32)
    for k in range(1, ks):
        s = (s + parts[k]).astype(np.float32)
    want_h = (h0 + s).astype(np.float32) if ks > 0 else h0
    np.testing.assert_array_equal(outs[0][0], want_h)
    if fmt == "none":
        return
    ref = op.rms_norm(want_h.astype(np.float64), nx.bf16_to_f64(w), 1e-6)
    if fmt == "f16":
        assert_f16_close(outs[0][1].astype(np.float64), ref, what="fused x")
        # the same bits through the separate residual add and norm entries
        h2 = dev(want_h)
        x2 = torch.empty((T, D), dtype=torch.float16, device="cuda")
        H.hr_rmsnorm(h2, T, D, dev_bf16(w), 1e-6, x2)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(x2.cpu().numpy(), outs[0][1])
    else:
        got = nx.e4m3_decode(outs[0][1])
        want = nx.e4m3_round(ref / a)
        diff = got != want
        assert diff.mean() < 1e-3
        step = np.abs(want) * 2.0 ** -3 + 2.0 ** -9
        assert np.all(np.abs(got - want)[diff] <= step[diff])


def test_linear_residual_is_deterministic(H):
    """A split-K residual projection (down at 13 and 512 rows) gives the same
    bits on every call."""
    import torch
    from gpu_util import dev, dev_bf16, dev_f16, log, seeded_f16
    for M in (13, 512):
        N, K = 2560, 9728
        log(f"residual determinism M={M}")
        x = dev_f16(seeded_f16((M, K), 77 + M, 1.0))
        w = dev_bf16(seeded_bf16((N, K), (12, M), 0.02))
        h0 = np.random.default_rng(M).standard_normal((M, N)).astype(np.float32)
        ws = H.linear_ws(H.HR_BF16, M, N, K, H.HR_EPI_RESIDUAL)
        assert ws is not None, "expected a split-K launch"
        res = []
        for _ in range(3):
            h = dev(h0.copy())
            H.hr_linear(x, w, None, 1.0, H.HR_BF16, M, N, K, H.HR_EPI_RESIDUAL, h, ws=ws)
            torch.cuda.synchronize()
            res.append(h.cpu().numpy())
        np.testing.assert_array_equal(res[0], res[1])
        np.testing.assert_array_equal(res[0], res[2])


# ----------------------------------------------------------------------------- A3
def _dims(H, m, causal=True):
    return H.make_dims(m.hidden, m.n_q_heads, m.n_kv_heads, m.head_dim, m.ffn, m.n_layers, m.rope_theta,
                       m.rms_eps, causal)


@pytest.mark.parametrize("model,lens,starts,slots,cap", [
    (synth.QWEN3_4B, [13], [0], [0], 2048),
    (synth.QWEN3_4B, [5, 1, 9], [0, 1500, 3], [2, 0, 1], 2048),
    (synth.TINY, [6, 20], [0, 40], [1, 0], 64),
])
def test_qknorm_rope_kv(H, model, lens, starts, slots, cap):
    import torch
    from gpu_util import BF16_NAN, bits_of, dev, dev_bf16, f64_of, log, poisoned_bf16, poisoned_f16
    m = model
    log(f"qknorm_rope_kv {m.name} lens={lens} starts={starts}")
    T = sum(lens)
    Hq, Hkv, d = m.n_q_heads, m.n_kv_heads, m.head_dim
    qkv = np.random.default_rng(20 + T + d).standard_normal((T, m.qkv_rows)).astype(np.float32)
    qw = seeded_bf16((d,), (21, d), 0.1, 1.0)
    kw = seeded_bf16((d,), (22, d), 0.1, 1.0)
    n_slots = max(slots) + 1
    kc, vc = poisoned_bf16((n_slots * cap, Hkv, d)), poisoned_bf16((n_slots * cap, Hkv, d))
    q_out = poisoned_f16((T, Hq, d))
    b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), starts, slots)
    H.hr_qknorm_rope_kv(_dims(H, m), b, dev(qkv), dev_bf16(qw), dev_bf16(kw), q_out,
                        H.make_kv(kc, vc, cap, n_slots))
    torch.cuda.synchronize()
    x = qkv.astype(np.float64)
    cu = b.h_cu
    kcb, vcb = bits_of(kc), bits_of(vc)
    written = np.zeros(n_slots * cap, bool)
    for s in range(len(lens)):
        a, e = cu[s], cu[s + 1]
        pos = starts[s] + np.arange(lens[s])
        q = op.apply_rope(op.rms_norm(x[a:e, :Hq * d].reshape(-1, Hq, d), nx.bf16_to_f64(qw)), pos, m.rope_theta)
        k = op.apply_rope(op.rms_norm(x[a:e, Hq * d:(Hq + Hkv) * d].reshape(-1, Hkv, d), nx.bf16_to_f64(kw)), pos,
                          m.rope_theta)
        rows = slots[s] * cap + pos
        written[rows] = True
        from gpu_util import assert_bf16_close, assert_f16_close
        assert_f16_close(f64_of(q_out[a:e]), q, abs_=1e-5, what="q")
        assert_bf16_close(nx.bf16_to_f64(kcb[rows]), k, abs_=1e-5, what="k cache")
        # v: the fp32 projection rounded once to bf16 (nearest even)
        np.testing.assert_array_equal(vcb[rows], nx.f32_to_bf16(qkv[a:e, (Hq + Hkv) * d:]).reshape(-1, Hkv, d))
    assert np.all(kcb[~written] == BF16_NAN) and np.all(vcb[~written] == BF16_NAN)


# ------------------------------------------------------------------ A3 + A4 fused (short prompts)
# Every sequence from position 0 with at most 32 rows: the cache must hold the
# bits hr_qknorm_rope_kv writes (the same arithmetic), and the output must be
# the attention of the q it produces over those keys (oracle on the fp16 q, bf16 k,
# v, as for hr_attention).  Cases: one 13-token prompt; a packed batch with a
# 1-row and a full 32-row prompt in permuted cache slots; the tiny model (d 64,
# 2 query heads per kv head); non-causal used keys with pads (their K/V left
# unwritten) and an e4m3 output.
@pytest.mark.parametrize("model,lens,slots,causal,used,fp8", [
    (synth.QWEN3_4B, [13], [0], True, None, False),
    (synth.QWEN3_4B, [1, 32, 7], [2, 0, 1], True, None, False),
    (synth.TINY, [6, 20], [1, 0], True, None, False),
    (synth.QWEN3_4B, [13, 20], [0, 1], False, [10, 20], True),
])
def test_qknorm_rope_attention(H, model, lens, slots, causal, used, fp8):
    import torch
    from gpu_util import BF16_NAN, bits_of, dev, dev_bf16, f64_of, log, poisoned_bf16, poisoned_f16
    m = model
    log(f"qknorm_rope_attention {m.name} lens={lens} causal={causal} fp8={fp8}")
    T, n, cap = sum(lens), len(lens), 40
    Hq, Hkv, d = m.n_q_heads, m.n_kv_heads, m.head_dim
    qkv = dev(np.random.default_rng(23 + T + d).standard_normal((T, m.qkv_rows)).astype(np.float32))
    qw = dev_bf16(seeded_bf16((d,), (24, d), 0.1, 1.0))
    kw = dev_bf16(seeded_bf16((d,), (25, d), 0.1, 1.0))
    b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), [0] * n, slots, used)
    dims = _dims(H, m, causal)
    caches = [(poisoned_bf16((n * cap, Hkv, d)), poisoned_bf16((n * cap, Hkv, d))) for _ in range(2)]
    out_scale = 0.01
    otype = H.HR_FP8_E4M3 if fp8 else H.HR_F16
    outs = [torch.full((T, Hq * d), 0x7F, dtype=torch.uint8, device="cuda") if fp8 else
            torch.full((T, Hq * d), float("nan"), dtype=torch.float16, device="cuda") for _ in range(2)]
    H.hr_qknorm_rope_attention(dims, b, qkv, qw, kw, H.make_kv(*caches[0], cap, n), outs[0], otype, out_scale)
    q_out = poisoned_f16((T, Hq, d))
    kv1 = H.make_kv(*caches[1], cap, n)
    H.hr_qknorm_rope_kv(dims, b, qkv, qw, kw, q_out, kv1)
    H.hr_attention(dims, b, q_out, kv1, outs[1], otype, out_scale)
    torch.cuda.synchronize()
    for c0, c1 in zip(*caches):
        np.testing.assert_array_equal(bits_of(c0), bits_of(c1))
    kcb = bits_of(caches[0][0])
    if not causal:      # pad rows past the used keys keep the poison
        for s in range(n):
            assert np.all(kcb[slots[s] * cap + used[s]:slots[s] * cap + cap] == BF16_NAN)
    if fp8:
        got = nx.e4m3_decode(outs[0].cpu().numpy()).reshape(T, Hq, d) * out_scale
    else:
        got = f64_of(outs[0]).reshape(T, Hq, d)
    assert np.all(np.isfinite(got))
    qv = f64_of(q_out)
    kv_, vv = f64_of(caches[1][0]), f64_of(caches[1][1])
    cu = b.h_cu
    grp = Hq // Hkv
    for s in range(n):
        a, e = cu[s], cu[s + 1]
        nk = lens[s] if causal else used[s]
        vis = (np.arange(nk)[None, :] <= np.arange(lens[s])[:, None]) if causal else np.ones((lens[s], nk), bool)
        rows = slice(slots[s] * cap, slots[s] * cap + nk)
        for hh in range(Hq):
            g = hh // grp
            ref = op.attention(qv[a:e, hh], kv_[rows, g], vv[rows, g], vis)
            err = np.abs(got[a:e, hh] - ref)
            if fp8:
                assert np.all(err <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -9 * out_scale + 2e-3), (s, hh, float(err.max()))
            else:
                assert np.all(err <= 2.0 ** -10 * np.abs(ref) + 2e-3), (s, hh, float(err.max()))


# ----------------------------------------------------------------------------- A4
@pytest.mark.parametrize("Hq,Hkv,d,lens,starts,causal,used", [
    (32, 8, 128, [13], [0], True, None),
    (32, 8, 128, [200, 7, 64], [0, 0, 30], True, None),
    (4, 2, 64, [6, 70], [0, 10], True, None),
    (8, 8, 64, [33], [0], True, None),
    (32, 8, 128, [100], [0], False, [90]),
    # causal rows of 4+ tiles on a short grid (the head split, two wave groups)
    (32, 8, 128, [512], [0], True, None),
    (32, 8, 128, [300, 129], [0, 50], True, None),
    # one row per sequence (decode steps: the decode kernel, one chunk per row)
    (32, 8, 128, [1, 1, 1], [0, 700, 2000], True, None),
    (4, 2, 64, [1, 1], [5, 130], True, None),
    (8, 8, 64, [1], [300], True, None),
    (32, 8, 128, [1, 1], [0, 0], False, [1, 1]),
])
def test_attention(H, Hq, Hkv, d, lens, starts, causal, used):
    _attention_case(H, Hq, Hkv, d, lens, starts, causal, used)


# key-chunked attention: (chunk_tiles, n_slots) forcing one-tile chunks, chunks
# lengthened by the slot cap (a 9-tile row with 2 slots), rows continuing a
# cached prefix, non-causal used keys with a short last chunk, fp8 output
@pytest.mark.parametrize("Hq,Hkv,d,lens,starts,causal,used,ct,slots,fp8", [
    (32, 8, 128, [512], [0], True, None, 2, 4, False),
    (32, 8, 128, [300], [0], True, None, 1, 8, False),
    (32, 8, 128, [544], [0], False, [512], 3, 3, False),
    (32, 8, 128, [544], [0], False, [530], 2, 2, False),
    (4, 2, 64, [200, 7, 90], [0, 0, 600], True, None, 2, 3, False),
    (8, 8, 64, [130], [0], True, None, 1, 64, False),
    (32, 8, 128, [256], [0], True, None, 1, 4, True),
    # decode steps cut into chunks and merged: one-tile chunks up to the slot
    # cap (a 32-tile row over 16 slots: 2-tile chunks), a row shorter than one
    # chunk written directly beside split ones, a ragged last chunk, GQA 2 and 1
    (32, 8, 128, [1, 1, 1], [0, 700, 2000], True, None, 1, 16, False),
    (32, 8, 128, [1, 1, 1, 1], [63, 64, 1000, 2046], True, None, 4, 4, True),
    (4, 2, 64, [1, 1], [60, 900], True, None, 2, 8, False),
    (8, 8, 64, [1, 1], [129, 1500], True, None, 3, 64, False),
])
def test_attention_chunked(H, Hq, Hkv, d, lens, starts, causal, used, ct, slots, fp8):
    _attention_case(H, Hq, Hkv, d, lens, starts, causal, used, chunked=(ct, slots), fp8=fp8)


# attention from fp16 copies of the keys and values (the layer's path for
# 385-1024 rows from position 0): the copies built here from the same bf16
# rows (widened exactly), every sequence at a batch row that is a multiple of
# 8.  Cases: the P = 512 prompt (8 pairs of query blocks); four sequences with
# odd and even block counts; a ragged last block with an e4m3 output and a
# larger row count of the copies; head dim 64 with 2 query heads per kv head;
# long rows with one query head per kv head; non-causal over the used keys
# (the FP8 prompt shape, and one used key).
@pytest.mark.parametrize("Hq,Hkv,d,lens,causal,used,fp8,tp_extra", [
    (32, 8, 128, [512], True, None, False, 0),
    (32, 8, 128, [296, 128, 40, 8], True, None, False, 0),
    (32, 8, 128, [100], True, None, True, 64),
    (4, 2, 64, [72, 33], True, None, False, 0),
    (8, 8, 64, [1000], True, None, False, 0),
    (32, 8, 128, [544], False, [512], False, 0),
    (32, 8, 128, [96, 64], False, [90, 1], False, 0),
])
def test_attention_f16(H, Hq, Hkv, d, lens, causal, used, fp8, tp_extra):
    _attention_case(H, Hq, Hkv, d, lens, [0] * len(lens), causal, used, fp8=fp8, f16_tp_extra=tp_extra)


def _attention_case(H, Hq, Hkv, d, lens, starts, causal, used, chunked=None, fp8=False, f16_tp_extra=None):
    import torch
    from gpu_util import dev_bf16, dev_f16, f64_of, log, seeded_f16
    log(f"attention Hq={Hq} Hkv={Hkv} d={d} lens={lens} causal={causal} chunked={chunked} fp8={fp8}")
    cap = max(s + l for s, l in zip(starts, lens)) + 3
    n = len(lens)
    T = sum(lens)
    q = seeded_f16((T, Hq, d), 30 + T * Hq + d, 1.0)
    kc = seeded_bf16((n * cap, Hkv, d), (31, cap, Hkv, d), 1.0)
    vc = seeded_bf16((n * cap, Hkv, d), (32, cap, Hkv, d), 1.0)
    b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), starts, list(range(n)), used)
    dims = H.make_dims(Hq * d, Hq, Hkv, d, 256, 1, 1e6, 1e-6, causal)
    kc_d, vc_d = dev_bf16(kc), dev_bf16(vc)
    kvd = H.make_kv(kc_d, vc_d, cap, n)
    out_scale = 0.01
    if fp8:
        out = torch.full((T, Hq * d), 0x7F, dtype=torch.uint8, device="cuda")      # e4m3 NaN
    else:
        out = torch.full((T, Hq * d), float("nan"), dtype=torch.float16, device="cuda")
    otype = H.HR_FP8_E4M3 if fp8 else H.HR_F16
    if chunked:
        ct, slots = chunked
        nb = H.hr_attention_chunked_workspace_bytes(dims, T, slots)
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device="cuda")
        H.hr_attention_chunked(dims, b, dev_f16(q), kvd, out, ct, slots, ws, otype, out_scale)
    elif f16_tp_extra is not None:
        # batch row t of sequence s is its key row t - cu[s]: cache row s cap + t - cu[s]
        Tp = (T + 31) // 32 * 32 + f16_tp_extra
        k16 = np.zeros((Tp, Hkv, d), np.float16)
        v16 = np.zeros((Tp, Hkv, d), np.float16)
        cu0 = np.concatenate([[0], np.cumsum(lens)])
        for s_ in range(n):
            rows = slice(s_ * cap, s_ * cap + lens[s_])
            k16[cu0[s_]:cu0[s_ + 1]] = nx.bf16_to_f64(kc[rows]).astype(np.float16)
            v16[cu0[s_]:cu0[s_ + 1]] = nx.bf16_to_f64(vc[rows]).astype(np.float16)
        H.hr_attention_f16(dims, b, dev_f16(q), dev_f16(k16), dev_f16(v16), Tp, out, otype, out_scale)
    else:
        H.hr_attention(dims, b, dev_f16(q), kvd, out, otype, out_scale)
    torch.cuda.synchronize()
    if fp8:
        got = nx.e4m3_decode(out.cpu().numpy()).reshape(T, Hq, d) * out_scale
    else:
        got = f64_of(out).reshape(T, Hq, d)
    qv, kv_, vv = q.astype(np.float64), nx.bf16_to_f64(kc), nx.bf16_to_f64(vc)
    cu = b.h_cu
    grp = Hq // Hkv
    for s in range(n):
        a, e = cu[s], cu[s + 1]
        pos = starts[s] + np.arange(lens[s])
        if causal:
            nk = starts[s] + lens[s]
            vis = np.arange(nk)[None, :] <= pos[:, None]
        else:
            nk = used[s]
            vis = np.ones((lens[s], nk), bool)
        for hh in range(Hq):
            g = hh // grp
            ref = op.attention(qv[a:e, hh], kv_[s * cap:s * cap + nk, g], vv[s * cap:s * cap + nk, g], vis)
            err = np.abs(got[a:e, hh] - ref)
            # fp16 output: half an ulp (2^-11 relative) plus the fp16 probabilities
            # of P V (2^-11 relative each, at most 2^-11 max|v| in the mean)
            if fp8:     # e4m3 keeps 3 mantissa bits: half a step of 2^-3 relative
                assert np.all(err <= 2.0 ** -4 * np.abs(ref) + 2.0 ** -9 * out_scale + 2e-3), (s, hh, float(err.max()))
            else:
                assert np.all(err <= 2.0 ** -10 * np.abs(ref) + 2e-3), (s, hh, float(err.max()))


# ----------------------------------------------------------------------------- A9 final + A10
@pytest.mark.parametrize("model,lens", [(synth.QWEN3_4B, [13]), (synth.QWEN3_4B, list(range(1, 34))),
                                        (synth.TINY, [6, 3])])
def test_head_logits(H, model, lens):
    import torch
    from gpu_util import dev, dev_bf16, log
    m = model
    log(f"head logits {m.name} n_seq={len(lens)}")
    D, N = m.hidden, m.n_codebooks * m.cb_vocab
    T = sum(lens)
    h = (np.random.default_rng(len(lens)).standard_normal((T, D)) * 5).astype(np.float32)
    wf = synth.final_norm(m)
    wh = synth.head_weight(m)
    b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), [0] * len(lens), list(range(len(lens))))
    out = torch.full((len(lens), N), float("nan"), device="cuda")
    ws = torch.empty(H.hr_head_workspace_bytes(len(lens), D), dtype=torch.uint8, device="cuda")
    H.hr_head_logits(dev(h), b, D, dev_bf16(wf), 1e-6, dev_bf16(wh), m.n_codebooks, m.cb_vocab, out, ws)
    torch.cuda.synchronize()
    z = op.rms_norm(h.astype(np.float64)[b.h_cu[1:] - 1], nx.bf16_to_f64(wf), 1e-6)
    ref = op.head_logits(z, nx.bf16_to_f64(wh), m.n_codebooks, m.cb_vocab).reshape(len(lens), N)
    got = out.cpu().numpy().astype(np.float64)
    scale = np.sqrt(np.sum(z ** 2, 1))[:, None] * np.sqrt(np.sum(nx.bf16_to_f64(wh) ** 2, 1))[None, :]
    assert np.all(np.abs(got - ref) <= 1e-5 * scale), float(np.abs(got - ref).max())


# ----------------------------------------------------------------------------- FP8 weight packing
def test_quantize_weight_bit_exact(H):
    import torch
    from gpu_util import dev_bf16
    N, K = 300, 2560
    wb = seeded_bf16((N, K), (40,), 0.02)
    wb[7] = 0                                   # a zero row: scale 1, codes 0
    w8 = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty(N, dtype=torch.float32, device="cuda")
    H.hr_quantize_weight_e4m3(dev_bf16(wb), N, K, w8, sc)
    torch.cuda.synchronize()
    s_ref, c_ref = of.weight_scales_e4m3(nx.bf16_to_f32(wb))
    np.testing.assert_array_equal(sc.cpu().numpy(), s_ref)
    got = w8.cpu().numpy()
    np.testing.assert_array_equal(nx.e4m3_decode(got), nx.e4m3_decode(c_ref))
