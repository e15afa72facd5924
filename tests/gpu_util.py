"""Helpers for the GPU parity tests: moving seeded bf16 bit patterns to the device
and back, NaN poisoning, comparison metrics.  No method arithmetic here."""
from __future__ import annotations

import sys

import numpy as np
import torch

BF16_NAN = 0x7FC0
F16_NAN = 0x7E00


def log(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(msg, file=sys.stderr, flush=True)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def dev_f16(a: np.ndarray) -> torch.Tensor:
    """float16 array (values already rounded by numpy, nearest even) -> device."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to("cuda")


def seeded_f16(shape, seed, std=1.0) -> np.ndarray:
    """Seeded normal draws rounded to fp16 (the activation format of the bf16-weight band)."""
    return (np.random.default_rng(seed).standard_normal(shape) * std).astype(np.float16)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def bits_of(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (host)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of_bf16(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


f64_of = f64_of_bf16      # any float tensor (bf16, fp16, fp32) -> float64 host array


def poisoned_bf16(shape) -> torch.Tensor:
    return torch.full(shape, BF16_NAN, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def poisoned_f16(shape) -> torch.Tensor:
    return torch.full(shape, F16_NAN, dtype=torch.int16, device="cuda").view(torch.float16)


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def assert_bf16_close(got, ref, rel=2.0 ** -8, abs_=1e-6, what=""):
    """|got - ref| <= rel |ref| + abs_ elementwise: a bf16 store (half-ulp 2^-9
    relative) of a value computed in fp32."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + abs_
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                           f"worst err {float(err.max()):.3g}")


def assert_f16_close(got, ref, rel=2.0 ** -10, abs_=1e-7, what=""):
    """An fp16 store (half-ulp 2^-11 relative; 2^-25 absolute in the subnormal
    range) of a value computed in fp32."""
    assert_bf16_close(got, ref, rel=rel, abs_=abs_, what=what)
