"""CPU oracle for the dequantise-fused skinny GEMV (test infrastructure only).

A plain, slow, obviously-correct implementation of what the GPU path computes,
written from the subject pages and the public definitions of the number
encodings. Only the tests, the package's smoke check and the benchmark's CPU
baseline may import it; the library never does, and nothing here imports the
library or its sources.

The pages this follows:
  * NInfer article ("单卡 LLM 推理引擎 NInfer 完全解析"), section 2 (custom CUDA
    operators and mixed quantised weights): decode is bound by weight reads,
    and per-format fused kernels do matmul, residual add and SwiGLU in one
    pass; groupwise Q4/Q5 and NVFP4 weights.
  * Decapybara page (GitHub - giveen/Decapybara), CUDA kernel list: a blocked
    NVFP4 GEMV and a top-8 softmax MoE router.
  * RustingStrata page, format list (Q8_0-style symmetric int8) and the note
    that run-to-run reordering of floating-point work causes divergence.

Modules
  encodings  exact and vectorised fp16 / bf16 / E4M3 / E2M1 codecs
  quant      per-format quantisers (logical codes and scale fields)
  layout     byte-exact device layout: pack and unpack
  dequant    logical fields -> fp32 weights (the bit-exact dump definition)
  gemv       fp64 reference GEMV, SwiGLU, MoE index / combine, tolerances

Parity status: every function is pinned by tests under tests/ (closed forms,
brute force in exact rationals, hand-worked blocks in tests/golden, special
cases). Agreement with the pages' own engines is "parity unpinned": the pages
print no bit layout, test vector or kernel-level figure.
"""
from . import encodings, quant, layout, dequant, gemv  # noqa: F401

FORMATS = {"int4": 1, "int5": 2, "int8": 3, "nvfp4": 4}
