"""Launches for the HBM-traffic counters of the dominant kernel (run it under
rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE):

  * the gate/up + SwiGLU GEMM at M=512 (512 x 19456 x 2560, bf16), once on each
    of 3 distinct weight matrices (so no launch finds its weights in the MALL
    from the one before);
  * a plain device copy of 256 MiB, twice: its counter reading against the
    bytes it must move calibrates the counters.

    python -m codebook_decode_amd.traffic_probe
"""
from __future__ import annotations

import sys


def main() -> None:
    import torch
    from . import hr as H
    H.lib()
    M, D, F = 512, 2560, 9728
    x = (torch.randn((M, D), device="cuda") * 0.5).to(torch.bfloat16)
    ws = [(torch.randn((2 * F, D), device="cuda") * 0.02).to(torch.bfloat16) for _ in range(3)]
    out = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    src = torch.empty(128 << 20, dtype=torch.bfloat16, device="cuda").fill_(1.0)   # 256 MiB
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for w in ws:
        H.hr_linear(x, w, None, 1.0, H.HR_BF16, M, 2 * F, D, H.HR_EPI_SWIGLU, out)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("gate/up x3, copy 256 MiB x2: done", file=sys.stderr)


if __name__ == "__main__":
    main()
