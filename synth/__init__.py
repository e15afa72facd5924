"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module only *draws* inputs: token ids, bf16 weight bit patterns, varlen
lengths, logits and decode state.  It holds none of the method's arithmetic
(no norm, no projection, no attention, no argmax), so the oracle and the HIP
path can both take their inputs from here without sharing any computation.

Every tensor is drawn from numpy's PCG64 seeded by a ``SeedSequence`` whose
entropy is ``[1234, model_key, layer, tensor_id, block]``: a tensor is cut into
blocks of ``BLOCK`` elements and each block has its own stream, so any block
(e.g. the embedding rows a prompt touches) can be drawn alone and blocks can be
drawn on several threads.  Values are float32 normals, scaled and shifted in
float32, then rounded to bfloat16 bit patterns with round-to-nearest-even.

The distributions follow the workloads stated for this hot path: weights and
embeddings N(0, 0.02); RMSNorm weights 1 + N(0, 0.1); token ids uniform over the
vocabulary; codebook logits N(0, 2) in bf16 with the end-of-codebook id forced
strictly top-1 in a fraction of rows.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

ROOT_SEED = 1234
BLOCK = 1 << 22          # elements per independently seeded block
SEED_IDS = 42            # prompt token ids
SEED_CALIB = 7           # the fixed FP8 calibration prompt
SEED_LENGTHS = 2024      # varlen prompt lengths
SEED_LOGITS = 99         # codebook-step logits
SEED_STATE = 5           # codebook-step initial frame counters
SEED_SAMPLING = 42       # per-stream sampling settings and generator keys

# tensor ids inside a model's seed space
T_EMBED, T_IN_NORM, T_POST_NORM, T_Q_NORM, T_K_NORM = 0, 1, 2, 3, 4
T_QKV, T_O, T_GU, T_DOWN = 5, 6, 7, 8
T_FINAL_NORM, T_HEAD, T_CB_EMBED = 9, 10, 11
NO_LAYER = 65535


@dataclass(frozen=True)
class Model:
    """Shapes of a Qwen3-style decoder with a multi-codebook audio head."""
    name: str
    key: int                 # seed-space id of the weights
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_layers: int
    vocab: int
    n_codebooks: int
    cb_vocab: int
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    @property
    def qkv_rows(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def attn_width(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def bos_id(self) -> int:      # the last two codebook ids are BOS and EOC
        return self.cb_vocab - 2

    @property
    def eoc_id(self) -> int:
        return self.cb_vocab - 1

    def with_layers(self, n: int) -> "Model":
        return replace(self, n_layers=n)


# d=256 single-layer model with a 4 x 130 codebook head
TINY = Model("tiny_d256", key=0, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
             ffn=768, n_layers=1, vocab=4096, n_codebooks=4, cb_vocab=130)
# 4B-class layer: d=2560, 32/8 heads of 128, SwiGLU 9728, 36 layers, 8 x 1026 head
QWEN3_4B = Model("qwen3_4b_d2560", key=1, hidden=2560, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, ffn=9728, n_layers=36, vocab=151936,
                 n_codebooks=8, cb_vocab=1026)


@dataclass
class Workload:
    """One named workload of the hot path, with its sizes."""
    name: str
    model: Model
    prompt_lens: tuple               # per sequence
    causal: bool = True
    capacity: int = 2048             # KV positions per cache slot
    padded_rows: int = 0             # >0: the single prompt is padded to this many rows
    fp8: bool = False
    frames: int = 0                  # decode frames driven after prefill (tiny model)
    cb_batch: int = 0                # codebook-step streams
    cb_steps: int = 0
    extra: dict = field(default_factory=dict)


def workloads() -> dict:
    lens = tuple(int(x) for x in varlen_lengths(32, 6, 256))
    return {
        "tiny_d256_p6": Workload("tiny_d256_p6", TINY, (6,), capacity=64, frames=8),
        "layer_d2560_p6": Workload("layer_d2560_p6", QWEN3_4B.with_layers(1), (6,)),
        "layer_d2560_p13": Workload("layer_d2560_p13", QWEN3_4B.with_layers(1), (13,)),
        "stack36_d2560_p13": Workload("stack36_d2560_p13", QWEN3_4B, (13,)),
        "stack36_d2560_p128": Workload("stack36_d2560_p128", QWEN3_4B, (128,)),
        "stack36_d2560_p512": Workload("stack36_d2560_p512", QWEN3_4B, (512,)),
        "fp8_layer_d2560_p512_pad544": Workload(
            "fp8_layer_d2560_p512_pad544", QWEN3_4B.with_layers(1), (512,), causal=False,
            capacity=544, padded_rows=544, fp8=True, extra={"calib_len": 32}),
        "varlen32_stack36_d2560": Workload("varlen32_stack36_d2560", QWEN3_4B, lens,
                                           capacity=256, cb_batch=64, cb_steps=16),
    }


# --------------------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------- drawing
def _stream(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *key])))


def _fill_block(out16: np.ndarray, key: tuple, b: int, std: float, mean: float,
                lo: int, hi: int) -> None:
    """Draw block ``b`` of a tensor and store elements [lo, hi) of it (block-local)."""
    n = hi - lo
    tmp = np.empty(hi, dtype=np.float32)
    _stream(*key, b).standard_normal(out=tmp, dtype=np.float32)
    v = tmp[lo:hi]
    v *= np.float32(std)
    if mean:
        v += np.float32(mean)
    out16[:n] = f32_to_bf16_bits(v)


def normal_bf16(shape, key: tuple, std: float, mean: float = 0.0,
                threads: int | None = None, out: np.ndarray | None = None) -> np.ndarray:
    """A seeded N(mean, std) tensor as bf16 bit patterns (uint16), drawn blockwise."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(n, dtype=np.uint16)
    flat = out.reshape(-1)
    assert flat.size == n
    nblk = (n + BLOCK - 1) // BLOCK
    jobs = [(b, b * BLOCK, min(n, (b + 1) * BLOCK)) for b in range(nblk)]

    def run(job):
        b, s, e = job
        _fill_block(flat[s:e], key, b, std, mean, 0, e - s)

    threads = threads or min(16, os.cpu_count() or 1)
    if nblk == 1 or threads == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    return out.reshape(shape)


def normal_bf16_rows(shape2d, rows: np.ndarray, key: tuple, std: float,
                     mean: float = 0.0) -> np.ndarray:
    """Rows ``rows`` of a seeded [R, C] tensor, identical to ``normal_bf16`` rows,
    drawing only the blocks that hold them."""
    R, C = shape2d
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, C), dtype=np.uint16)
    cache: dict = {}
    for i, r in enumerate(rows):
        assert 0 <= r < R
        s = int(r) * C
        e = s + C
        pos = 0
        while s < e:
            b = s // BLOCK
            if b not in cache:
                blk_len = min(R * C, (b + 1) * BLOCK) - b * BLOCK
                tmp = np.empty(blk_len, dtype=np.uint16)
                _fill_block(tmp, key, b, std, mean, 0, blk_len)
                cache[b] = tmp
            take = min(e, (b + 1) * BLOCK) - s
            off = s - b * BLOCK
            out[i, pos:pos + take] = cache[b][off:off + take]
            pos += take
            s += take
    return out


# --------------------------------------------------------------------------- model tensors
def layer_tensors(m: Model, layer: int) -> dict:
    """bf16 bit patterns of one decoder layer, row-major [out, in].

    ``w_qkv`` rows are q heads, then k heads, then v heads; ``w_gu`` rows are
    the gate projection, then the up projection.
    """
    D, d = m.hidden, m.head_dim
    k = lambda t: (m.key, layer, t)
    return {
        "in_norm": normal_bf16((D,), k(T_IN_NORM), 0.1, 1.0),
        "post_norm": normal_bf16((D,), k(T_POST_NORM), 0.1, 1.0),
        "q_norm": normal_bf16((d,), k(T_Q_NORM), 0.1, 1.0),
        "k_norm": normal_bf16((d,), k(T_K_NORM), 0.1, 1.0),
        "w_qkv": normal_bf16((m.qkv_rows, D), k(T_QKV), 0.02),
        "w_o": normal_bf16((D, m.attn_width), k(T_O), 0.02),
        "w_gu": normal_bf16((2 * m.ffn, D), k(T_GU), 0.02),
        "w_down": normal_bf16((D, m.ffn), k(T_DOWN), 0.02),
    }


def final_norm(m: Model) -> np.ndarray:
    return normal_bf16((m.hidden,), (m.key, NO_LAYER, T_FINAL_NORM), 0.1, 1.0)


def head_weight(m: Model) -> np.ndarray:
    return normal_bf16((m.n_codebooks * m.cb_vocab, m.hidden), (m.key, NO_LAYER, T_HEAD), 0.02)


def codebook_embed(m: Model) -> np.ndarray:
    return normal_bf16((m.n_codebooks * m.cb_vocab, m.hidden), (m.key, NO_LAYER, T_CB_EMBED), 0.02)


def embed_table(m: Model) -> np.ndarray:
    return normal_bf16((m.vocab, m.hidden), (m.key, NO_LAYER, T_EMBED), 0.02)


def embed_rows(m: Model, ids: np.ndarray) -> np.ndarray:
    return normal_bf16_rows((m.vocab, m.hidden), ids, (m.key, NO_LAYER, T_EMBED), 0.02)


# --------------------------------------------------------------------------- prompts, batches
def prompt_ids(m: Model, n: int, seq: int = 0, seed: int = SEED_IDS) -> np.ndarray:
    """``n`` token ids uniform over the vocabulary (int32)."""
    g = _stream(seed, m.key, n, seq)
    return g.integers(0, m.vocab, n, dtype=np.int64).astype(np.int32)


def calibration_ids(m: Model, n: int = 32) -> np.ndarray:
    """The fixed seeded calibration prompt used for the static FP8 scales."""
    return prompt_ids(m, n, seq=0, seed=SEED_CALIB)


def varlen_lengths(n: int, lo: int, hi: int, seed: int = SEED_LENGTHS) -> np.ndarray:
    """``n`` prompt lengths uniform over [lo, hi] (inclusive)."""
    return _stream(seed, n, lo, hi).integers(lo, hi + 1, n, dtype=np.int64).astype(np.int32)


def packed_batch(lens, capacity: int, start_pos=None, cache_slot=None) -> dict:
    """A packed varlen batch: ``cu_seqlens`` and per-sequence cache placement."""
    lens = np.asarray(lens, dtype=np.int32)
    n = lens.size
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    sp = np.zeros(n, np.int32) if start_pos is None else np.asarray(start_pos, np.int32)
    cs = np.arange(n, dtype=np.int32) if cache_slot is None else np.asarray(cache_slot, np.int32)
    return {"cu_seqlens": cu, "start_pos": sp, "cache_slot": cs,
            "max_seqlen": int(lens.max()) if n else 0, "capacity": capacity}


# --------------------------------------------------------------------------- codebook step
def codebook_logits(B: int, K: int, V: int, step: int, eoc_id: int, eoc_frac: float = 0.05,
                    std: float = 2.0, seed: int = SEED_LOGITS) -> np.ndarray:
    """bf16 bit patterns [B, K, V]: N(0, std) logits with the EOC id forced strictly
    top-1 (row max + 1.0) in about ``eoc_frac`` of the (b, k) rows."""
    g = _stream(seed, B, K, V, step)
    x = g.standard_normal((B, K, V), dtype=np.float32) * np.float32(std)
    bits = f32_to_bf16_bits(x).reshape(B, K, V)
    force = g.random((B, K)) < eoc_frac
    vals = bf16_bits_to_f32(bits)
    rowmax = vals.max(axis=2)
    bumped = f32_to_bf16_bits((rowmax + np.float32(1.0)).astype(np.float32))
    bits[force, eoc_id] = bumped[force]
    return bits


def codebook_state(B: int, K: int, frame_hi: int = 16, seed: int = SEED_STATE) -> dict:
    """Initial per-stream decode state: frame counters uniform over [0, frame_hi),
    no codebook has emitted EOC yet, no stream done."""
    g = _stream(seed, B, K)
    return {"frame": g.integers(0, frame_hi, B, dtype=np.int64).astype(np.int32),
            "eoc_seen": np.zeros((B, K), np.uint8),
            "done": np.zeros(B, np.uint8)}


def sampling_settings(B: int, seed: int = SEED_SAMPLING, serving: bool = False) -> dict:
    """Per-stream sampling settings: temperature fp32, top_k int32, top_p fp32 and
    a 64-bit generator key (uint64) per stream.  ``serving``: every stream at
    temperature 1, top-k 50, top-p 0.95 (the serving runs' settings); else a mix
    that covers greedy (T = 0), top-k off / 1 / 50 / 200 / all, top-p off / 0.95 / 0.5 / 0
    and temperatures 0.7 / 1.0 / 1.3."""
    g = _stream(seed, B, 1 if serving else 0)
    keys = g.integers(0, 2 ** 63, B, dtype=np.int64).astype(np.uint64) * np.uint64(2) + \
        g.integers(0, 2, B, dtype=np.int64).astype(np.uint64)
    if serving:
        return {"temperature": np.ones(B, np.float32), "top_k": np.full(B, 50, np.int32),
                "top_p": np.full(B, 0.95, np.float32), "seed": keys}
    i = np.arange(B)
    return {"temperature": np.array([0.0, 0.7, 1.0, 1.3], np.float32)[i % 4],
            "top_k": np.array([0, 1, 50, 200, 1 << 20], np.int32)[i % 5],
            "top_p": np.array([1.0, 0.95, 0.5, 0.95, 0.0, 0.95, 1.0], np.float32)[i % 7],
            "seed": keys}
