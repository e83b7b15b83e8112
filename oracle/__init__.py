"""CPU oracle for the 4-bit block-quantized MoE layer with a bf16 LoRA adapter.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The HIP library never calls it, and this package imports nothing from
the HIP library or its Python binding: the two share no code, tables or
constants.  Only the seeded input generators in ``synth/`` feed both.

What each module follows (page titles and sections of the source pages):

* ``formats``  - the number formats: E2M1 values, E4M3 block scales, bf16, and
  the NF4 codebook ("Getting GLM-5.2 NVFP4 Post-Training off the ground",
  section "Why can't we just transpose the one copy?"; "nf4moe - QLoRA for a
  743B Fused-MoE", section "The fix: dequant-on-forward for routed experts").
* ``quant``    - NVFP4 rowwise quantization with a per-tensor or per-row FP32
  scale and the Four-Over-Six choice per 16-block ("The 4-bitter Lesson",
  sections "Method" and "Four-Over-Six for RL Weights and Activations"), its
  dequantization, and NF4 blocksize-64 absmax quantization ("nf4moe", same
  section).
* ``routing``  - softmax top-k routing and the stable expert permutation
  ("nf4moe", the QuantizedNaiveMoe forward: expert_mask / expert_hit).
* ``moe``      - the routed-expert forward, the dgrad through DQ(Q(W)) and the
  LoRA weight gradients, in float64 ("Getting GLM-5.2 ...", section "The 4-bit
  base that was actually using 8-bit memory"; "The 4-bitter Lesson", section
  "Improving Gradient Stability"; "nf4moe", the module's forward).

Floating-point conventions: the quantizers use numpy float32 elementwise
operations (each one IEEE round-to-nearest-even operation, never fused), so
every rounding is reproducible bit for bit.  The GEMM chains use float64.

Parity status: every function is pinned by ``tests/test_oracle_*.py`` except
the exact numeric values of the NF4 codebook, which the pages name but never
print: parity unpinned for those 16 values (their construction and its
invariants are pinned).
"""
