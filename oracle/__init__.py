"""CPU oracle for the FP8 prefill matmul path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy/Python implementations of every step of
the path, written from the pages (realizar 0.8.4 source pages
``cublas_prefill/gemm.rs`` and ``cublas_prefill/mod.rs``) and from the public
GGUF K-quant block formats.  Floating point is done in float64 (exact where
the arithmetic allows it) and rounded once to float32 where the path has an
fp32 result.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``fp8_prefill_gemm_amd``) and imports nothing from it; the GPU path never
imports it.

Modules:
  e4m3     — the bitwise FP32 -> E4M3 encoder and the OCP E4M3FN decoder
  kquant   — Q4_K / Q6_K super-block dequantisation to fp32
  fp8_path — absmax, scales, weight packing, activation quantisation,
             exact FP8 GEMM, fused epilogue and the parity error bound
  kquant_gemv — the small-M GEMV straight from K-quant blocks (fp32 input
             and output) and its fp32-accumulation error bound

Parity status: every function is pinned by tests under ``tests/`` that do
not re-derive it (fixed points, closed forms, exhaustive sweeps, a library
cross-check and brute force).  One reading is unpinned: that the Q4_K/Q6_K
field layout equals the public GGUF layout (the pages never print the
dequant kernels, and no GGUF file is available); this is "parity unpinned"
with respect to real GGUF files only — GPU-vs-oracle parity does not depend
on it.
"""
