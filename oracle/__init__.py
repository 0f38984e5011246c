"""CPU oracle for the QLoRA linear layer and gated MLP (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, fp64 statement of what the GPU library
computes. It exists to check the HIP path, never to serve it: only the test
suite, the smoke check and the CPU-baseline leg of the benchmark may import
it. The HIP library shares no code, header, table or helper with it; the only
thing both sides consume is the seeded synthetic input produced by
``qlora_fine_tuning_amd.inputs``.

Modules
-------
nf4    : the 4-bit NormalFloat level table, quantizer, packing and the
         bit-exact dequantization contract.
qlora  : QLoRA linear forward/backward, gated-MLP forward/backward
         (SwiGLU and tanh-GeGLU), q/k/v on one input, the matmul-chain FLOP
         counter.
fast_kernels : RMS layernorm, RoPE embeddings and the cross-entropy loss,
         forward and backward (the pages' other hand-derived kernels).

Sources (the pages this follows):
- "Unsloth update: Mistral support and performance improvements"
  (dbyun.net/tutorial/10039): benchmark configuration block (QLoRA nf4 on
  q/k/v/o/gate/up/down, rank 16, alpha 16, dropout 0), the per-optimisation
  breakdown, and items 10-11 "manual autograd" with the chained-matmul
  bracketing analysis.
- "Show HN: 80% faster, 50% less memory, 0% loss of accuracy Llama
  finetuning": hand-derived backprop, "0% loss in accuracy - all exact".
- "Fine-tuning Gemma with Unsloth" (dbyun.net/tutorial/10042), section
  "GeGLU vs SwiGLU activation".
- Reddit talk summary (llminfo.tech/posts/1fk0acj): fused LoRA, SwiGLU
  kernel, chained matrix multiplication.

Parity status: every function here is pinned by tests under ``tests/``
(closed forms, special cases that reduce to torch/scipy routines, finite
differences, the pages' printed bracketing ratios). The one point left
unpinned is agreement of the NF4 level table with bitsandbytes' table, whose
values are not on the pages ("parity unpinned" for that comparison only).
"""
