"""CPU oracle for the scaled low-precision GEMM and routed fused-MoE path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links this code; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, tables or
constants with the HIP library: every codec, every quantisation step and every
GEMM here is written out from the definitions on the source pages (and the OCP
FP8 / MX format definitions they rely on), in numpy, with float64 accumulation.

Sources (cited by title and section throughout):

* "vLLM PR 50949 review" -- per-expert-block BRGEMM / TinyGEMM dispatch for the
  CPU FP8 / MXFP4 routed fused-MoE (the ``moe_fp8.cpp`` and ``gemm.h`` listings,
  implementation items 1-4).
* "SGLang PR 32618 review" -- CPU per-tensor FP8 W8A16 GEMM
  ``fp8_per_tensor_scaled_mm_cpu`` (implementation items 1-2, the ``fp8.py`` and
  ``test_gemm.py`` listings).
* "SGLang PR 35605 review" -- block-wise FP8 W8A8 linear on XPU through
  ``scaled_mm`` (the ``fp8_utils.py`` listing, implementation items 1 and 3, the
  ``test_xpu_fp8_linear.py`` listing).

Modules:

* ``codecs``  -- e4m3 / e2m1 / e8m0 / bf16 encode and decode.
* ``quant``   -- per-token 1x128 group quantisation to e4m3.
* ``dense``   -- per-tensor W8A16 GEMM and block-scaled W8A8 / W8A16 linears.
* ``align``   -- expert sort / block alignment of routed rows.
* ``moe``     -- routed fused-MoE experts (FP8 block and MXFP4 weights).
* ``mx``      -- MXFP8 quantisation (e4m3 + e8m0 per 32) and the MX-scaled linear
  (MXFP8 activations x MXFP8 / MXFP4 weights).

Every function has at least one pin in ``tests/test_oracle_*.py`` that checks
it against something other than itself (library routines, closed forms,
brute force, invariants).  The one unpinned piece is the exponential inside
SiLU (host libm vs device math): only the bf16 tolerance covers it.
"""

from . import codecs, quant, dense, align, moe, mx  # noqa: F401
