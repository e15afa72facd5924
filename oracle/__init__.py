"""CPU oracle for the batched Qwen3-style prefill and the delayed-codebook step.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP library (``codebook_decode_amd``) never imports it and this
package imports nothing from the HIP library: the two share no kernels, headers,
helpers, tables or constants.  Inputs come from ``synth`` (seeded draws only).

Everything is plain NumPy in float64 unless a step's precision is part of the
contract (the codebook-embedding sum, which is an fp32 sum in codebook order
rounded to bf16).  Sources, cited by page title and section:

* "Stabilize Higgs Audio termination and prefill" (FlashRT pull request 141),
  Summary and Root cause: the kernelised batched prefill (embedding lookup,
  projection GEMMs, q/k norm + RoPE, KV writes) and the delayed-codebook helper
  (per-frame argmax, delay handling, codebook-embedding accumulation), with the
  delayed-EOC check covering every codebook.
* "feat(higgs-audio): add checkpoint loading and validation foundation"
  (pegainfer pull request 864), Summary / What changed: a Qwen3 text backbone
  prefill feeding an audio-head projection.
* flashrt-structures 0.2.0, ``prefill_tower/fp8_chain.py`` (module docstring,
  ``_build_rope``, ``_prefill_mask_facts``, the quantiser table built in
  ``_quantize`` and the per-call ``run`` of ``_make_run``): RMSNorm with eps
  1e-6, rotate-half RoPE, attention over exactly the used keys, static
  per-tensor activation scales ``amax / FP8_MAX``.
* vLLM-Omni pull request 8226 (Higgs Audio v3 streaming on Model Runner V2),
  Purpose and Test Plan: temperature / top-k / top-p sampling of the codebook
  rows with per-request seeded exponential noise.

Modules: ``numerics`` (bf16 widen/round, e4m3 codec), ``prefill`` (layer, stack,
head), ``codebook`` (delayed-codebook step), ``fp8`` (weight/activation scales,
calibration, fake-quant layer), ``sampling`` (Philox4x64-10 noise and the row
sampler), ``policy`` (the step with sampling and the termination policies).
"""
from . import numerics, prefill, codebook, fp8, sampling, policy  # noqa: F401
