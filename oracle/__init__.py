"""CPU oracle for one NVFP4 routed-MoE layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the layer
computes: the e2m1 / e4m3 / bf16 codecs, the NVFP4 activation quantizer, the
sigmoid top-k routing, the permutation metadata, the two grouped GEMMs with the
gated activation and requantization between them, the post-expert finalize,
the converted weight layout with its expert-TP slice views, and the rel-L2
probe. It follows the four pages this project is built from:

  * "vllm.models.muse_spark.nvidia.specialized_decode.runtime.expert_tp"
    (the expert_tp page: slice views, route rows, the rel-L2 probe);
  * "vllm.models.muse_spark.nvidia.specialized_decode.runtime.flashinfer_ops"
    (the flashinfer_ops page: the routed experts op, its metadata, gemm2_rows);
  * "vllm.models.muse_spark.nvidia.muse_moe_runner" (the runner page: scalar
    folding, the post-expert finalize);
  * "vllm.models.muse_spark.nvidia.model" (the model page: the router, the
    input quantization).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import anything here. The GPU path never imports, links or calls it, and
it imports nothing from the GPU path: the only code both sides use is the
seeded input generator, which holds none of the method's arithmetic.

Floating point is fp64 unless the pages fix the precision. Where a float
decides an integer (a quantized code, a top-k choice) the decision is taken in
fp32, the kernels' precision, with the op order stated in each function.

Pins: every function is checked in ``tests/test_oracle_*.py`` against things
other than itself (exact rational brute force, closed forms, invariants,
special cases that reduce to textbook routines). Functions without such a pin
say "parity unpinned" here; there are none at present.
"""
