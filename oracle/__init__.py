"""CPU oracle for the Fast-dLLM block-cache decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The GPU library never calls it, and it imports nothing from the GPU library: the two
share only the seeded input generators in ``synth``.

It is a plain, slow, step-by-step NumPy implementation of what the method computes,
written from the pages that describe Fast-dLLM:

* the ccyt168.com Fast-dLLM article, section 1.1 "Block-Wise KV Cache" (DualCache
  caches prompt prefix and masked suffix; adjacent steps' KV are nearly identical)
  and section 1.2 "Confidence-Aware Parallel Decoding" (confidence is the probability
  the model gives a token; only tokens at or above a threshold such as 0.9 are decoded
  in parallel, the rest wait; the (n+1)eps <= 1 theorem for greedy decoding);
* the techwalker.com explainer "Fast-dLLM: NVIDIA researchers accelerate diffusion
  LLMs without training via KV cache and parallel decoding", section "Core
  innovation: a KV cache suited to diffusion models" (two-step block cache: before a
  block, compute and keep the other blocks' KV; after it, recompute all KV; DualCache)
  and section "Solving the quality loss of parallel decoding" (threshold instead of a
  fixed token count).

Floating point runs in float64 unless a caller asks for float32.  bf16 models round
to bf16 (nearest even, via fp32) at the storage points listed in ``model.py``.

Parity status per function (what pins it) is listed in each module's header.
"""
