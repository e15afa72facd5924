"""hr_codebook_step_policy on the GPU against the oracle.

* Greedy (no policy, or temperature 0 everywhere): bit-exact with hr_codebook_step.
* Sampled rows (temperature / top-k / top-p / seeded Philox race) on the
  batched workload (64 streams, 8 x 1026, bf16 and fp32 logits, EOC forced
  top-1 in 5% of rows): each sampled code equals the oracle's, except on rows
  where a float decision came within the tolerance of its threshold (the top-p
  bar or the race's top two scores); there the GPU's code must be a valid
  choice, and the oracle continues with it.  Everything else (codes, frame,
  EOC flags, done, aligned frames, embedding sums, end frames, guard state) is
  bit-exact.
* The sampled codes' distribution: 16384 rows of one logits row under the
  serving settings (T 1, top-k 50, top-p 0.95), empirical frequencies against
  the renormalised probabilities.
* Termination policies: the hand-worked traces and a long seeded run with the
  cascade and the stop guard on.
"""
import json
import os

import numpy as np
import pytest

import synth
from oracle import numerics as nx
from oracle import policy as opol
from oracle import sampling as osm

pytestmark = pytest.mark.gpu

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sampling_cases.json")
# Rows too close to call in fp32.  top-p bar: |mass ahead - p S| / S below TOL_P
# (an fp32 sum of up to 1026 softmax terms is good to ~1e-6 of S); race: the
# winner's score within TOL_RACE of the runner-up (scores below 20 in magnitude,
# fp32 logs good to ~1e-6)
TOL_P = 1e-5
TOL_RACE = 1e-5


@pytest.fixture(scope="module")
def H():
    import codebook_decode_amd.hr as H
    H.lib()
    return H


class GpuStreams:
    """Device state of B streams plus the policy arrays."""

    def __init__(self, H, B, K, V, D, st, E_bits, max_frames, params=None, cascade=False, repeat_limit=0):
        import torch
        from gpu_util import dev, dev_bf16
        self.H, self.B, self.K, self.V, self.D, self.maxf = H, B, K, V, D, max_frames
        self.frame, self.seen, self.done = dev(st["frame"].copy()), dev(st["eoc_seen"].copy()), dev(st["done"].copy())
        self.aligned = dev(np.full((B, max_frames, K), -1, np.int32))
        self.codes = torch.empty((B, K), dtype=torch.int32, device="cuda")
        self.emb = torch.empty((B, D), dtype=torch.bfloat16, device="cuda")
        self.E = dev_bf16(E_bits)
        self.end = dev(np.full(B, -1, np.int32))
        self.last = dev(np.full((B, K), -1, np.int32))
        self.run = dev(np.zeros(B, np.int32))
        p = params or {}
        self.pol = H.make_policy(
            temperature=dev(p["temperature"]) if "temperature" in p else None,
            top_k=dev(p["top_k"]) if "top_k" in p else None,
            top_p=dev(p["top_p"]) if "top_p" in p else None,
            seed=dev(p["seed"].view(np.int64)) if "seed" in p else None,
            eoc_cascade=cascade, repeat_limit=repeat_limit,
            end_frame=self.end if (cascade or repeat_limit) else None,
            last_codes=self.last if repeat_limit else None,
            repeat_run=self.run if repeat_limit else None)

    def step(self, d_logits, policy=True):
        import torch
        from gpu_util import bits_of
        bos, eoc = self.V - 2, self.V - 1
        self.H.hr_codebook_step_policy(self.B, self.K, self.V, bos, eoc, d_logits, self.frame, self.seen, self.done,
                                       self.codes, self.aligned, self.maxf, self.E, self.D, self.emb,
                                       self.pol if policy else None)
        torch.cuda.synchronize()
        return self.codes.cpu().numpy().copy(), bits_of(self.emb).copy()

    def state(self):
        return {k: getattr(self, k).cpu().numpy().copy()
                for k in ("frame", "seen", "done", "aligned", "end", "last", "run")}


def _setup(B, K, V, D, seed):
    rng = np.random.default_rng(seed)
    E_bits = nx.f32_to_bf16((rng.standard_normal((K * V, D)) * 0.5).astype(np.float32))
    return E_bits, nx.bf16_to_f32(E_bits)


@pytest.mark.parametrize("f32", [False, True])
def test_greedy_policy_is_the_plain_step(H, f32):
    """No policy and temperature 0 give hr_codebook_step's codes, bit for bit."""
    import torch
    from gpu_util import log, dev, dev_bf16, bits_of
    B, K, V, D, steps, maxf = 64, 8, 1026, 64, 6, 12
    E_bits, _ = _setup(B, K, V, D, 3)
    st = synth.codebook_state(B, K)
    log(f"greedy policy vs plain step f32={f32}")
    plain = GpuStreams(H, B, K, V, D, st, E_bits, maxf)
    nopol = GpuStreams(H, B, K, V, D, st, E_bits, maxf)
    zeroT = GpuStreams(H, B, K, V, D, st, E_bits, maxf,
                       params={"temperature": np.zeros(B, np.float32), "seed": np.arange(B, dtype=np.uint64)})
    for s in range(steps):
        lg = synth.codebook_logits(B, K, V, 100 + s, V - 1, eoc_frac=0.2)
        d_lg = dev(nx.bf16_to_f32(lg)) if f32 else dev_bf16(lg)
        H.hr_codebook_step(B, K, V, V - 2, V - 1, d_lg, plain.frame, plain.seen, plain.done, plain.codes,
                           plain.aligned, maxf, plain.E, D, plain.emb)
        torch.cuda.synchronize()
        c0, e0 = plain.codes.cpu().numpy().copy(), bits_of(plain.emb).copy()
        c1, e1 = nopol.step(d_lg, policy=False)
        c2, e2 = zeroT.step(d_lg)
        for c, e in ((c1, e1), (c2, e2)):
            np.testing.assert_array_equal(c, c0, err_msg=f"codes step {s}")
            np.testing.assert_array_equal(e, e0, err_msg=f"emb step {s}")
    for g in (nopol, zeroT):
        a, b = plain.state(), g.state()
        for k in ("frame", "seen", "done", "aligned"):
            np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def _check_sampled_step(lg32, gpu_codes, o_state, params, cascade, repeat_limit, E, V, maxf):
    """Oracle step with teacher forcing on rows too close to call; returns the
    oracle's (codes, emb) and the count of such rows."""
    frame, seen, done, aligned, end, last, run = o_state
    probe = [a.copy() for a in (frame, seen, done, aligned, end, last, run)]
    _, _, info = opol.codebook_step_policy(
        lg32, probe[0], probe[1], probe[2], V - 2, V - 1, E, probe[3], maxf, temperature=params["temperature"],
        top_k=params["top_k"], top_p=params["top_p"], seed=params["seed"], eoc_cascade=cascade,
        repeat_limit=repeat_limit, end_frame=probe[4], last_codes=probe[5], repeat_run=probe[6])
    B, K, _ = lg32.shape
    choices = np.full((B, K), -1, np.int32)
    close = 0
    for b in range(B):
        for k in range(K):
            inf = info[b][k]
            if inf is None:
                continue
            if inf["p_margin"] >= TOL_P and inf["race_margin"] >= TOL_RACE:
                continue                      # the oracle's own choice stands
            close += 1
            g = int(gpu_codes[b, k])
            T, tk, tp = float(params["temperature"][b]), int(params["top_k"][b]), float(params["top_p"][b])
            wide, narrow = osm.relaxed_kept(lg32[b, k], T, tk, tp, TOL_P)
            assert wide[g], f"stream {b} codebook {k}: code {g} outside the kept set"
            sc = inf["scores"]
            # the race within tolerance of the best narrowly kept score
            full = np.where(wide, lg32[b, k].astype(np.float64) / T -
                            np.log(-np.log(osm.row_uniforms(int(params["seed"][b]), int(frame[b]), k, V))),
                            -np.inf)
            best_narrow = np.max(np.where(narrow, full, -np.inf))
            assert full[g] >= best_narrow - TOL_RACE, (b, k, g, full[g], best_narrow, sc.max())
            choices[b, k] = g
    codes, emb, _ = opol.codebook_step_policy(
        lg32, frame, seen, done, V - 2, V - 1, E, aligned, maxf, temperature=params["temperature"],
        top_k=params["top_k"], top_p=params["top_p"], seed=params["seed"], eoc_cascade=cascade,
        repeat_limit=repeat_limit, end_frame=end, last_codes=last, repeat_run=run, choices=choices)
    return codes, emb, close


@pytest.mark.parametrize("f32", [False, True])
def test_sampled_workload_vs_oracle(H, f32):
    from gpu_util import log, dev, dev_bf16
    m = synth.QWEN3_4B
    B, K, V, D, steps, maxf = 64, m.n_codebooks, m.cb_vocab, 128, 5, 24
    E_bits, E = _setup(B, K, V, D, 9)
    st = synth.codebook_state(B, K)
    params = synth.sampling_settings(B)
    cascade, limit = True, 3
    log(f"sampled workload B={B} K={K} V={V} f32={f32}")
    g = GpuStreams(H, B, K, V, D, st, E_bits, maxf, params=params, cascade=cascade, repeat_limit=limit)
    o = [st["frame"].copy(), st["eoc_seen"].copy(), st["done"].copy(), np.full((B, maxf, K), -1, np.int32),
         np.full(B, -1, np.int32), np.full((B, K), -1, np.int32), np.zeros(B, np.int32)]
    close_total = sampled = 0
    for s in range(steps):
        bits = synth.codebook_logits(B, K, V, 200 + s, V - 1)
        lg32 = nx.bf16_to_f32(bits)
        if f32:
            lg32 = (lg32 + np.random.default_rng(s).standard_normal(lg32.shape).astype(np.float32) * 1e-3)
            lg32 = lg32.astype(np.float32)
        d_lg = dev(lg32) if f32 else dev_bf16(bits)
        gc, ge = g.step(d_lg)
        oc, oe, close = _check_sampled_step(lg32, gc, o, params, cascade, limit, E, V, maxf)
        close_total += close
        sampled += int(np.sum(params["temperature"] > 0)) * K
        np.testing.assert_array_equal(gc, oc, err_msg=f"codes step {s}")
        np.testing.assert_array_equal(ge, oe, err_msg=f"emb step {s}")
    gs = g.state()
    for name, ref in zip(("frame", "seen", "done", "aligned", "end", "last", "run"), o):
        np.testing.assert_array_equal(gs[name], ref, err_msg=name)
    log(f"rows too close to call: {close_total} of {sampled}")
    assert close_total <= max(4, sampled // 10), (close_total, sampled)


def test_serving_settings_distribution(H):
    """16384 draws of one row (2048 streams x 8 codebooks, one step each) under
    T 1 / top-k 50 / top-p 0.95: frequencies against the kept set's renormalised
    probabilities, Pearson chi-square below its mean + 6 standard deviations."""
    import torch
    from gpu_util import log, dev, dev_bf16
    B, K, V, D = 2048, 8, 1026, 8
    row = synth.codebook_logits(1, 1, V, 7, V - 1, eoc_frac=0.0)[0, 0]
    bits = np.broadcast_to(row, (B, K, V)).copy()
    params = synth.sampling_settings(B, serving=True)
    st = {"frame": np.full(B, 20, np.int32), "eoc_seen": np.zeros((B, K), np.uint8), "done": np.zeros(B, np.uint8)}
    E_bits, _ = _setup(B, K, V, D, 1)
    log("serving-settings distribution B=2048")
    g = GpuStreams(H, B, K, V, D, st, E_bits, 4, params=params)
    codes, _ = g.step(dev_bf16(bits))
    x = nx.bf16_to_f32(row).astype(np.float64)
    _, info = osm.sample_row(x, 1.0, 50, float(np.float32(0.95)), np.full(V, 0.5))
    kept = info["kept"]
    p = np.zeros(V)
    q = np.exp(x[kept] - x[kept].max())
    p[kept] = q / q.sum()
    counts = np.bincount(codes.ravel(), minlength=V).astype(np.float64)
    assert np.all(counts[p == 0] == 0), "a code outside the kept set"
    pos = p > 0
    e = counts.sum() * p[pos]
    chi2 = np.sum((counts[pos] - e) ** 2 / e)
    dof = pos.sum() - 1
    assert chi2 < dof + 6 * np.sqrt(2 * dof), (chi2, dof)


def test_golden_termination_traces(H):
    from gpu_util import log, dev
    gold = json.load(open(GOLD))
    K, V, D = 4, 6, 8
    for tr in gold["traces"]:
        log(f"termination trace {tr['name']}")
        init = tr.get("init", {})
        st = {"frame": np.array([init.get("frame", 0)], np.int32),
              "eoc_seen": np.array([init.get("eoc_seen", [0] * K)], np.uint8), "done": np.zeros(1, np.uint8)}
        E_bits, _ = _setup(1, K, V, D, 2)
        g = GpuStreams(H, 1, K, V, D, st, E_bits, 16, cascade=bool(tr["eoc_cascade"]),
                       repeat_limit=tr["repeat_limit"])
        if "last_codes" in init:
            g.last.copy_(dev(np.array([init["last_codes"]], np.int32)))
            g.run.copy_(dev(np.array([init["repeat_run"]], np.int32)))
        for s, am in enumerate(tr["argmax"]):
            lg = np.zeros((1, K, V), np.float32)
            for k in range(K):
                lg[0, k, am[k]] = 9.0
            codes, _ = g.step(dev(lg))
            assert codes[0].tolist() == tr["codes"][s], (tr["name"], s)
            st_ = g.state()
            assert int(st_["end"][0]) == tr["end_frame"][s], (tr["name"], s)
            assert int(st_["done"][0]) == tr["done"][s], (tr["name"], s)


def test_cascade_and_guard_long_run(H):
    """64 greedy streams over 40 steps whose logits repeat in runs (so the guard
    fires) with EOC top-1 in some rows (so the cascade fires): bit-exact."""
    from gpu_util import log, dev
    B, K, V, D, steps, maxf = 64, 8, 130, 32, 40, 48
    E_bits, E = _setup(B, K, V, D, 4)
    st = synth.codebook_state(B, K)
    limit = 4
    log("cascade + guard long run")
    g = GpuStreams(H, B, K, V, D, st, E_bits, maxf, cascade=True, repeat_limit=limit)
    o = [st["frame"].copy(), st["eoc_seen"].copy(), st["done"].copy(), np.full((B, maxf, K), -1, np.int32),
         np.full(B, -1, np.int32), np.full((B, K), -1, np.int32), np.zeros(B, np.int32)]
    rng = np.random.default_rng(31)
    lg = rng.integers(0, 50, (B, K, V)).astype(np.float32)
    for s in range(steps):
        change = rng.random(B) < 0.25                 # a quarter of the streams get new rows each step
        lg[change] = rng.integers(0, 50, (int(change.sum()), K, V)).astype(np.float32)
        eoc_rows = rng.random((B, K)) < 0.01
        lg[eoc_rows, V - 1] = 99.0
        gc, ge = g.step(dev(lg))
        oc, oe, _ = opol.codebook_step_policy(lg, o[0], o[1], o[2], V - 2, V - 1, E, o[3], maxf, eoc_cascade=True,
                                              repeat_limit=limit, end_frame=o[4], last_codes=o[5], repeat_run=o[6])
        np.testing.assert_array_equal(gc, oc, err_msg=f"codes step {s}")
        np.testing.assert_array_equal(ge, oe, err_msg=f"emb step {s}")
        lg[eoc_rows, V - 1] = 0.0
    gs = g.state()
    for name, ref in zip(("frame", "seen", "done", "aligned", "end", "last", "run"), o):
        np.testing.assert_array_equal(gs[name], ref, err_msg=name)
    assert (o[4] >= 0).sum() > 8 and o[2].sum() > 4      # both rules fired and streams finished
