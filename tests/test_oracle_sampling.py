"""Pins of the sampling and termination-policy oracle (no GPU).

* Philox4x64-10 against NumPy's own Philox bit generator (a library routine),
  including the element-to-word layout of a row's noise.
* Kept sets (top-k, top-p, ties, p <= 0) against hand-worked cases in
  tests/golden/sampling_cases.json, and top-k against its counting form.
* The exponential race against the distribution it must produce: empirical
  frequencies over many seeded steps against the renormalised probabilities
  (a chi-square bound), at three temperatures and under top-k / top-p.
* The termination rules against hand-worked traces, and the special cases that
  reduce to the pinned greedy step.
"""
import json
import os

import numpy as np
import pytest

from oracle import codebook as ocb
from oracle import policy as opol
from oracle import sampling as osm

GOLD = os.path.join(os.path.dirname(__file__), "golden", "sampling_cases.json")


def _numpy_philox_block(counter, key):
    """First 4 words NumPy's Philox (4x64, 10 rounds) gives for a state whose
    counter is one below ``counter``: NumPy increments before it generates."""
    c = [int(w) for w in counter]
    c[0] -= 1
    for i in range(3):          # borrow
        if c[i] < 0:
            c[i] += 1 << 64
            c[i + 1] -= 1
    g = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
    return [int(v) for v in g.random_raw(4)]


@pytest.mark.parametrize("counter,key", [
    ((1, 0, 0, 0), (0, 0)),
    ((5, 7, 9, 11), (0x0123456789ABCDEF, 0xFEDCBA9876543210)),
    ((0, 1, 0, 0), (42, 0)),                                  # a borrow through word 0
    ((2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1), (2 ** 64 - 1, 2 ** 64 - 1)),
    ((123456789, 3, 77, 0), (2024, 0)),
])
def test_philox_matches_numpy(counter, key):
    got = osm.philox4x64([np.array([w], dtype=np.uint64) for w in counter], key)
    assert [int(w[0]) for w in got] == _numpy_philox_block(counter, key)


def test_row_uniforms_layout():
    seed, step, k, V = 987654321, 17, 3, 23
    u = osm.row_uniforms(seed, step, k, V)
    for v in range(V):
        word = _numpy_philox_block((step, k, v // 4, 0), (seed, 0))[v % 4]
        assert u[v] == ((word >> 41) + 0.5) / 2 ** 23


def test_uniform_range_and_float32_exact():
    w = np.array([0, 2 ** 41 - 1, 2 ** 41, 2 ** 63, 2 ** 64 - 1], dtype=np.uint64)
    u = osm.uniform_from_word(w)
    assert u[0] == 0.5 / 2 ** 23 and u[1] == u[0]
    assert u[2] == 1.5 / 2 ** 23
    assert u[3] == 0.5 + 0.5 / 2 ** 23
    assert u[4] == 1.0 - 0.5 / 2 ** 23
    r = osm.uniform_from_word(np.random.default_rng(5).integers(0, 2 ** 63, 1000, dtype=np.uint64) * 2)
    assert np.all((r > 0) & (r < 1)) and np.all(r.astype(np.float32).astype(np.float64) == r)


def test_golden_kept_sets():
    cases = json.load(open(GOLD))["kept_cases"]
    for c in cases:
        x = np.log(np.array(c["probs"], dtype=np.float64))
        _, info = osm.sample_row(x, 1.0, c["top_k"], c["top_p"], np.full(len(x), 0.5))
        assert list(info["kept"]) == c["kept"], c["name"]
        wide, narrow = osm.relaxed_kept(x, 1.0, c["top_k"], c["top_p"], 1e-9)
        assert list(np.nonzero(wide)[0]) == c["kept"] and list(np.nonzero(narrow)[0]) == c["kept"], c["name"]


def test_top_k_counting_form():
    """kept <=> fewer than k elements are strictly larger (ties at the k-th value stay)."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        V = int(rng.integers(2, 40))
        x = rng.integers(-4, 5, V).astype(np.float64)     # many ties
        k = int(rng.integers(1, V + 2))
        _, info = osm.sample_row(x, 1.0, k, 1.0, np.full(V, 0.5))
        expect = [v for v in range(V) if (k >= V) or np.sum(x > x[v]) < k]
        assert list(info["kept"]) == expect


def test_greedy_and_top1_ignore_noise():
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.normal(0, 2, 30)
        u = rng.uniform(0.01, 0.99, 30)
        assert osm.sample_row(x, 0.0, 50, 0.95, u)[0] == int(np.argmax(x))
        assert osm.sample_row(x, -1.0, 0, 1.0, u)[0] == int(np.argmax(x))
        assert osm.sample_row(x, 0.7, 1, 1.0, u)[0] == int(np.argmax(x))     # distinct values
        assert osm.sample_row(x, 1.3, 0, 0.0, u)[0] == int(np.argmax(x))


def _frequencies(x, T, top_k, top_p, n, seed=77, k=2):
    V = len(x)
    counts = np.zeros(V)
    for t in range(n):
        c, _ = osm.sample_row(x, T, top_k, top_p, osm.row_uniforms(seed, t, k, V))
        counts[c] += 1
    return counts


def _chi2_ok(counts, probs):
    """Pearson chi-square over the cells with positive probability; cells with
    zero probability must be empty.  Bound: mean + 6 standard deviations of the
    chi-square law (the draws are fixed by the seeds, so this is a fixed check)."""
    n = counts.sum()
    pos = probs > 0
    assert np.all(counts[~pos] == 0)
    e = n * probs[pos]
    chi2 = np.sum((counts[pos] - e) ** 2 / e)
    dof = pos.sum() - 1
    return chi2 < dof + 6 * np.sqrt(2 * dof), chi2


@pytest.mark.parametrize("T", [0.5, 1.0, 2.0])
def test_race_samples_the_softmax(T):
    x = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.5])
    p = np.exp(x / T) / np.exp(x / T).sum()
    counts = _frequencies(x, T, 0, 1.0, 6000)
    ok, chi2 = _chi2_ok(counts, p)
    assert ok, (chi2, counts / counts.sum(), p)


def test_race_samples_under_top_k_and_top_p():
    x = np.log(np.array([0.05, 0.35, 0.25, 0.15, 0.2]))
    # top-3 keeps {1, 2, 4}; top-p .7 then keeps {1, 2} (golden case top_k3_top_p)
    counts = _frequencies(x, 1.0, 3, 0.7, 5000)
    p = np.array([0, 0.35, 0.25, 0, 0]) / 0.6
    ok, chi2 = _chi2_ok(counts, p)
    assert ok, (chi2, counts)
    counts = _frequencies(x, 1.0, 3, 1.0, 5000)
    p = np.array([0, 0.35, 0.25, 0, 0.2]) / 0.8
    ok, chi2 = _chi2_ok(counts, p)
    assert ok, (chi2, counts)


def test_race_sign_mistake_would_fail():
    """The frequency check separates the race from its plausible mistakes."""
    x = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.5])
    p = np.exp(x) / np.exp(x).sum()
    V, n = len(x), 6000
    for wrong in (lambda z, E: z + np.log(E), lambda z, E: z - E, lambda z, E: z + E):
        counts = np.zeros(V)
        for t in range(n):
            E = -np.log(osm.row_uniforms(77, t, 2, V))
            counts[osm.argmax_lowest(wrong(x, E))] += 1
        assert not _chi2_ok(counts, p)[0]


def _trace_run(tr):
    K, V, bos, eoc = 4, 6, 4, 5
    D = 2
    E = np.zeros((K * V, D), dtype=np.float32)
    init = tr.get("init", {})
    frame = np.array([init.get("frame", 0)], dtype=np.int32)
    seen = np.array([init.get("eoc_seen", [0] * K)], dtype=np.uint8)
    done = np.zeros(1, dtype=np.uint8)
    end = np.array([init.get("end_frame", -1)], dtype=np.int32)
    last = np.array([init.get("last_codes", [-1] * K)], dtype=np.int32)
    run = np.array([init.get("repeat_run", 0)], dtype=np.int32)
    out = []
    for s, am in enumerate(tr["argmax"]):
        logits = np.zeros((1, K, V), dtype=np.float32)
        for k in range(K):
            logits[0, k, am[k]] = 9.0
        codes, _, _ = opol.codebook_step_policy(
            logits, frame, seen, done, bos, eoc, E, eoc_cascade=bool(tr["eoc_cascade"]),
            repeat_limit=tr["repeat_limit"], end_frame=end, last_codes=last, repeat_run=run)
        out.append((list(codes[0]), int(end[0]), int(done[0])))
    return out


def test_golden_termination_traces():
    for tr in json.load(open(GOLD))["traces"]:
        got = _trace_run(tr)
        for s, (codes, e, d) in enumerate(got):
            assert codes == tr["codes"][s], (tr["name"], s)
            assert e == tr["end_frame"][s], (tr["name"], s)
            assert d == tr["done"][s], (tr["name"], s)


def test_policy_off_and_greedy_is_the_plain_step():
    rng = np.random.default_rng(8)
    B, K, V, D = 6, 4, 12, 8
    E = rng.normal(0, 1, (K * V, D)).astype(np.float32)
    st1 = [np.array([0, 1, 3, 7, 2, 5], dtype=np.int32), np.zeros((B, K), np.uint8), np.zeros(B, np.uint8)]
    st2 = [a.copy() for a in st1]
    al1 = np.full((B, 10, K), -1, np.int32)
    al2 = al1.copy()
    for step in range(12):
        logits = rng.integers(0, 6, (B, K, V)).astype(np.float32)
        if step % 3 == 2:
            logits[:, :, V - 1] = 9.0                     # EOC rows
        c1, e1 = ocb.codebook_step(logits, *st1, V - 2, V - 1, E, al1, 10)
        c2, e2, _ = opol.codebook_step_policy(logits, *st2, V - 2, V - 1, E, al2, 10,
                                              temperature=np.zeros(B, np.float32))
        assert np.array_equal(c1, c2) and np.array_equal(e1, e2) and np.array_equal(al1, al2)
        for a, b in zip(st1, st2):
            assert np.array_equal(a, b)


def test_sampled_step_rows_use_their_own_counters():
    """Each (stream, step, codebook) row draws from its own counter: the sampled
    code of a row equals sample_row with row_uniforms(seed, frame, k)."""
    rng = np.random.default_rng(21)
    B, K, V, D = 3, 4, 40, 4
    E = rng.normal(0, 1, (K * V, D)).astype(np.float32)
    logits = rng.normal(0, 2, (B, K, V)).astype(np.float32)
    frame = np.array([3, 9, 4], np.int32)
    T = np.array([1.0, 0.8, 1.5], np.float32)
    seeds = np.array([1, 2 ** 40 + 5, 99], np.uint64)
    codes, _, info = opol.codebook_step_policy(
        logits, frame.copy(), np.zeros((B, K), np.uint8), np.zeros(B, np.uint8), V - 2, V - 1, E,
        temperature=T, top_k=np.array([50, 5, 0], np.int32), top_p=np.array([0.95, 1.0, 0.8], np.float32),
        seed=seeds)
    for b in range(B):
        for k in range(K):
            if frame[b] < k:
                continue
            expect, _ = osm.sample_row(logits[b, k], float(T[b]), [50, 5, 0][b], [0.95, 1.0, 0.8][b],
                                       osm.row_uniforms(int(seeds[b]), int(frame[b]), k, V))
            assert codes[b, k] == expect
