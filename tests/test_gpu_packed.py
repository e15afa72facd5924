"""Packed fp16 weights (HR_F16_PACKED, hr_pack_weight) on the GPU.

The packing is a layout change plus the conversion the bf16 kernels already
make in registers, so the packed path must reproduce the bf16 path bit for
bit: every projection (skinny and tiled configurations, each epilogue) and
whole layers, whose results the bf16 tests hold to the oracle.  The layout
itself is checked against a host rearrangement of numpy's round-to-nearest-
even fp16 conversion of the bf16 values, subnormal range included.
"""
import numpy as np
import pytest

import synth
from oracle import numerics as nx

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


def packed_reference(wbits: np.ndarray, gate_up: bool) -> np.ndarray:
    """Host layout of hr_pack_weight: [K/32][N][32] fp16 bit patterns; gate_up
    rows reordered so that packed row 64 p + 32 u + r holds row u F + 32 p + r."""
    N, K = wbits.shape
    f16 = nx.bf16_to_f32(wbits).astype(np.float16)
    rows = np.arange(N)
    if gate_up:
        F = N // 2
        rows = ((rows >> 5) & 1) * F + 32 * (rows >> 6) + (rows & 31)
    return f16[rows].reshape(N, K // 32, 32).transpose(1, 0, 2).copy().view(np.uint16)


def packed(H, dw, N, K, gate_up):
    import torch
    out = torch.full((N, K), float("nan"), dtype=torch.float16, device="cuda")
    H.hr_pack_weight(dw, N, K, gate_up, out)
    return out


@pytest.mark.parametrize("N,K,gate_up", [(192, 96, False), (128, 64, True), (19456 // 8, 2560, True),
                                         (2560, 9728 // 8, False)])
def test_pack_weight_layout(H, N, K, gate_up):
    from gpu_util import dev_bf16, log
    rng = np.random.default_rng(N + K)
    w = synth.normal_bf16((N, K), (70, N, K), 0.02)
    # magnitudes across the fp16 subnormal range and the largest finite values
    tiny = rng.integers(0, N * K, 64)
    w.reshape(-1)[tiny] = (nx.f32_to_bf16(np.float32(2.0) ** rng.integers(-30, -14, 64).astype(np.float32)
                                          * rng.choice([-1.0, 1.0], 64).astype(np.float32)))
    # (65280: the largest bf16 value below the fp16 overflow at 65520)
    w.reshape(-1)[tiny[:4]] = nx.f32_to_bf16(np.array([65280.0, -65280.0, 2.0 ** -24, -(2.0 ** -17)], np.float32))
    log(f"pack N={N} K={K} gate_up={gate_up}")
    got = packed(H, dev_bf16(w), N, K, gate_up).cpu().numpy().view(np.uint16).reshape(K // 32, N, 32)
    np.testing.assert_array_equal(got, packed_reference(w, gate_up))


def test_pack_weight_rejects_values_outside_fp16(H):
    from gpu_util import dev_bf16
    w = synth.normal_bf16((64, 64), (71,), 0.02)
    w[3, 5] = nx.f32_to_bf16(np.array([70000.0], np.float32))[0]
    with pytest.raises(H.HrError, match="fp16 range"):
        packed(H, dev_bf16(w), 64, 64, False)


# the 4B projections at the row counts that select each skinny / tiled
# configuration (M <= 16 skinny; 17-64, 65-128, 129-384, 385-1024, > 1024 tiles)
SHAPES = {"qkv": (6144, 2560, "F32"), "o": (2560, 4096, "RESIDUAL"), "gu": (19456, 2560, "SWIGLU"),
          "down": (2560, 9728, "RESIDUAL")}


@pytest.mark.parametrize("M", [1, 13, 16, 17, 64, 65, 128, 129, 200, 512, 1100])
@pytest.mark.parametrize("site", list(SHAPES))
def test_linear_packed_equals_bf16(H, site, M):
    import torch
    from gpu_util import dev_bf16, dev_f16, log, seeded_f16
    N, K, epi_name = SHAPES[site]
    epi = getattr(H, "HR_EPI_" + epi_name)
    log(f"packed linear {site} M={M}")
    x = dev_f16(seeded_f16((M, K), 7000 + M, 1.0))
    wb = dev_bf16(synth.normal_bf16((N, K), (72, N, K), 0.02))
    wp = packed(H, wb, N, K, site == "gu")
    outs = []
    for w, wtype in ((wb, H.HR_BF16), (wp, H.HR_F16_PACKED)):
        if epi == H.HR_EPI_SWIGLU:
            out = torch.full((M, N // 2), float("nan"), dtype=torch.float16, device="cuda")
        elif epi == H.HR_EPI_RESIDUAL:
            out = torch.from_numpy(np.random.default_rng(M).standard_normal((M, N)).astype(np.float32)).cuda()
        else:
            out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        H.hr_linear(x, w, None, 1.0, wtype, M, N, K, epi, out, ws=H.linear_ws(wtype, M, N, K, epi))
        outs.append(out)
    torch.cuda.synchronize()
    a, b = (o.cpu().numpy() for o in outs)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("lens,starts,slots,cap", [([13], [0], [0], 64), ([512], [0], [0], 1024),
                                                   ([40, 7, 130, 1], [0, 5, 0, 100], [0, 1, 2, 3], 256)],
                         ids=["p13", "p512", "varlen4_continuation"])
def test_layer_packed_equals_bf16(H, lens, starts, slots, cap):
    import torch
    from gpu_util import dev, log
    from model_util import dims_of, kv_cache, upload_layer, workspace
    m = synth.QWEN3_4B
    bits = synth.layer_tensors(m, 3)
    dl = upload_layer(bits)
    shapes = {"w_qkv": (m.qkv_rows, m.hidden), "w_o": (m.hidden, m.attn_width), "w_gu": (2 * m.ffn, m.hidden),
              "w_down": (m.hidden, m.ffn)}
    dp = H.pack_layer_weights(dl, shapes)
    dims = dims_of(H, m, True, 1)
    T = sum(lens)
    h0 = np.random.default_rng(T).standard_normal((T, m.hidden)).astype(np.float32)
    n_slots = max(slots) + 1
    res = []
    for layer, wtype in ((H.make_layer(dl), H.HR_BF16), (H.make_layer(dp, H.HR_F16_PACKED), H.HR_F16_PACKED)):
        log(f"layer wtype={wtype} lens={lens}")
        kc, vc = kv_cache(m, n_slots, cap, poison=False)
        b = H.Batch(np.concatenate([[0], np.cumsum(lens)]), starts, slots)
        h = dev(h0)
        H.hr_prefill_layer(dims, layer, b, h, H.make_kv(kc, vc, cap, n_slots), workspace(H, dims, wtype, T))
        torch.cuda.synchronize()
        res.append((h.cpu().numpy(), kc.cpu().view(torch.int16).numpy(), vc.cpu().view(torch.int16).numpy()))
    for a, b in zip(res[0], res[1]):
        np.testing.assert_array_equal(a, b)
