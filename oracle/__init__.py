"""Plain CPU oracle for the streamed NF4 + LoRA linear.

TEST INFRASTRUCTURE ONLY.  This package is the slow, obviously correct
reference that the HIP path is checked against.  Only the test suite, the
smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product library never does, and the oracle
imports nothing from the product package.  The two share no code: the only
common module is ``synthgen`` (seeded random inputs, no arithmetic of the
method).

Floating point is fp64 wherever the method leaves the precision open (GEMM
accumulations, LoRA products, gradients).  Where the format fixes a precision
(the fp32 code table, the fp32 absmax, the fp32 product and the bf16 rounding
of a decoded weight, the fp32 division and comparison inside quantization)
the oracle uses exactly that precision, through numpy float32 arithmetic,
which is IEEE round-to-nearest-even.

Modules
-------
nf4         code table, bf16 rounding, quantize / pack / decode
lora        LoRA linear forward and backward (plain matrix definitions)
stream_sim  the layer-stream schedule and its event log
layer       one decoder layer's projections composed into a layer step
head        embedding gather, token cross-entropy, sequence sums, sigmoid DPO
decoder     RMSNorm, RoPE, causal GQA attention, SwiGLU, a whole decoder layer and a
            whole-model SFT step, forward and hand-written backward
"""
