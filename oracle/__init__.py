"""CPU oracle for self-speculative decoding — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy implementation of what the GPU library computes:
a Llama-style decoder, layer-skipped / early-exit drafting with a confidence
stop, a full-depth verify pass that reuses the draft's KV cache, the
speculative accept/reject rule, SWIFT matchness scoring of candidate skip
masks, and greedy verification of confidence-sized draft trees.  It shares no code with the HIP library (the two only share the seeded
input generator in ``synth``) and is the parity authority for it.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import or call anything in this package; the product path never does.

Sources (web pages; cited by title and section):
  * "SWIFT: On-the-Fly Self-Speculative Decoding for LLM Inference Acceleration"
    (paper digest, paperlayer.ai, arXiv 2410.06916v2) — "SWIFT digest" below.
  * "ACL'24 | LayerSkip: Meta 把 Self-Speculative Decoding 从头训到尾" (blog,
    marsggbo.github.io) — "LayerSkip blog" below.
  * "SpecEE: Accelerating Large Language Model Inference with Speculative Early
    Exiting" (study notes, velog.io) — "SpecEE notes" below.

Parity pins for every function are in tests/test_oracle_*.py.  Functions whose
result has no independent pin say "parity unpinned" in their docstring.
"""
