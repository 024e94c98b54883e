"""CPU oracle for the software-pipelined tiled GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, loads or
calls it, and the two share no code.

Contents:
  gemm      -- the plain fp32-accumulating GEMM (C, via ctypes), NT and NN forms,
               and the binary16 / bfloat16 conversions it uses.
  timeline  -- the discrete-event copy->compute pipeline model.
  budget    -- the multi-buffered on-chip memory budget and the
               configuration-space pruning it implies.
  attention -- plain softmax attention (the KV-length loop), float64.
"""
