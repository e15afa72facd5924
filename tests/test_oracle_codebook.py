"""Pins of the delayed-codebook oracle: hand-derived cases (tests/golden) and
invariants of the delay pattern over many steps."""
import json
import os

import numpy as np
import torch

from oracle import codebook as oc
from oracle import numerics as nx

GOLD = os.path.join(os.path.dirname(__file__), "golden", "codebook_cases.json")


def load():
    with open(GOLD) as f:
        return json.load(f)


def index_rows(K, V):
    return np.stack([np.array([r, 0.5], np.float32) for r in range(K * V)])


def test_golden_cases_one_stream_each():
    g = load()
    K, V = g["K"], g["V"]
    E = index_rows(K, V)
    for c in g["cases"]:
        logits = np.array(c["logits"], np.float32)[None]
        frame = np.array([c["frame"]], np.int32)
        seen = np.array([c["eoc_seen"]], np.uint8)
        done = np.array([c["done"]], np.uint8)
        aligned = np.full((1, c["max_frames"], K), -1, np.int32)
        codes, emb = oc.codebook_step(logits, frame, seen, done, g["bos"], g["eoc"], E,
                                      aligned, c["max_frames"])
        assert codes[0].tolist() == c["codes"], c["name"]
        assert int(frame[0]) == c["frame_out"], c["name"]
        assert seen[0].tolist() == c["eoc_seen_out"], c["name"]
        assert int(done[0]) == c["done_out"], c["name"]
        want = np.full_like(aligned, -1)
        for f, k, v in c["aligned_writes"]:
            want[0, f, k] = v
        np.testing.assert_array_equal(aligned, want, err_msg=c["name"])
        assert nx.bf16_to_f64(emb[0]).tolist() == c["emb"], c["name"]


def test_golden_cases_as_one_batch():
    """Streams are independent: the cases batched together give the same answers."""
    g = load()
    K, V = g["K"], g["V"]
    cases = [c for c in g["cases"] if c["max_frames"] == 8]
    logits = np.array([c["logits"] for c in cases], np.float32)
    frame = np.array([c["frame"] for c in cases], np.int32)
    seen = np.array([c["eoc_seen"] for c in cases], np.uint8)
    done = np.array([c["done"] for c in cases], np.uint8)
    codes, _ = oc.codebook_step(logits, frame, seen, done, g["bos"], g["eoc"], index_rows(K, V))
    assert codes.tolist() == [c["codes"] for c in cases]
    assert frame.tolist() == [c["frame_out"] for c in cases]


def test_golden_embedding_rounding_ties_to_even():
    g = load()
    K, V = g["K"], g["V"]
    r = g["rounding"]
    E = np.zeros((K * V, 2), np.float32)
    for idx, row in r["rows"].items():
        E[int(idx)] = row
    codes, emb = oc.codebook_step(np.array(r["logits"], np.float32)[None], np.array([r["frame"]], np.int32),
                                  np.zeros((1, K), np.uint8), np.zeros(1, np.uint8), g["bos"], g["eoc"], E)
    assert codes[0].tolist() == r["codes"]
    assert nx.bf16_to_f64(emb[0]).tolist() == r["emb"]


def test_delay_pattern_invariants_over_many_steps():
    """aligned[f, k] is the code codebook k emitted at step f + k; BOS exactly
    while t < k; once done, everything is EOC and frozen; done <=> all seen."""
    rng = np.random.default_rng(21)
    B, K, V, steps, maxf = 6, 4, 11, 14, 16
    bos, eoc = V - 2, V - 1
    E = rng.standard_normal((K * V, 8)).astype(np.float32)
    frame = rng.integers(0, 3, B).astype(np.int32)
    start = frame.copy()
    seen = np.zeros((B, K), np.uint8)
    done = np.zeros(B, np.uint8)
    aligned = np.full((B, maxf, K), -1, np.int32)
    history = []
    for s in range(steps):
        lg = rng.standard_normal((B, K, V)).astype(np.float32)
        lg[rng.random((B, K)) < 0.25, eoc] = 10.0
        before_done = done.copy()
        f0 = frame.copy()
        codes, _ = oc.codebook_step(lg, frame, seen, done, bos, eoc, E, aligned, maxf)
        history.append((f0, before_done, codes.copy()))
        np.testing.assert_array_equal(done, np.all(seen == 1, axis=1).astype(np.uint8))
    for b in range(B):
        for f0, was_done, codes in history:
            if was_done[b]:
                assert np.all(codes[b] == eoc)
                continue
            t = int(f0[b])
            for k in range(K):
                if t < k:
                    assert codes[b, k] == bos
                elif t - k < maxf:
                    assert aligned[b, t - k, k] == codes[b, k]
        # once codebook k emitted EOC it never emits anything else
        for k in range(K):
            emitted = [codes[b, k] for f0, wd, codes in history]
            if eoc in emitted:
                first = emitted.index(eoc)
                assert all(x == eoc for x in emitted[first:])
        assert int(frame[b]) - int(start[b]) == sum(1 for _, wd, _ in history if not wd[b])


def test_argmax_lowest_index_matches_torch_first_occurrence():
    rng = np.random.default_rng(22)
    x = rng.integers(-3, 4, (500, 17)).astype(np.float32)     # many ties
    want = torch.from_numpy(x).argmax(dim=1).numpy()
    got = np.array([oc.argmax_lowest(r) for r in x])
    np.testing.assert_array_equal(got, want)


def test_embedding_sum_equals_exact_sum_when_fp32_partials_are_exact():
    """The fp32 k-order sum rounded once to bf16 equals the exactly rounded
    bf16 of the true sum whenever every fp32 partial sum is exact."""
    rng = np.random.default_rng(23)
    K, V, D = 8, 9, 64
    E_bits = nx.f32_to_bf16(rng.standard_normal((K * V, D)).astype(np.float32) * 0.02)
    E = nx.bf16_to_f32(E_bits)
    lg = rng.standard_normal((3, K, V)).astype(np.float32)
    frame = np.full(3, 20, np.int32)
    codes, emb = oc.codebook_step(lg, frame, np.zeros((3, K), np.uint8), np.zeros(3, np.uint8),
                                  V - 2, V - 1, E)
    checked = 0
    for b in range(3):
        rows = np.stack([E[k * V + codes[b, k]] for k in range(K)]).astype(np.float64)
        exact = np.sum(rows, axis=0)                                 # exact in float64 here
        partial32 = np.cumsum(rows.astype(np.float32), axis=0, dtype=np.float32)
        ok = np.all(partial32.astype(np.float64) == np.cumsum(rows, axis=0), axis=0)
        want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(emb[b][ok], want[ok])
        checked += int(ok.sum())
    assert checked > 100
