"""CPU oracle for the LLM.int8() mixed-precision outlier matmul.

TEST INFRASTRUCTURE ONLY: the test-suite, the package smoke check and the
benchmark's CPU-baseline leg are the only code allowed to import it.  The
product path (the HIP library and its Python binding) never imports, links
or calls anything here, and this package imports nothing from the product.

Every function follows the pages' definitions step by step in numpy, with
fp32-exact rounding where the method fixes an integer result and fp64 for
the floating-point output.  See llm_int8.py for the cited passages and the
readings taken where the pages are ambiguous.

Pins (in tests/, none of which re-type the oracle's formulas):
  * brute force on tiny inputs (pure-Python loops, Python integers, exact
    rationals) for every step;
  * alpha = +inf reduces to plain vector-wise int8 (no fp16 path);
  * alpha = 0 reduces to the exact fp16 matmul (numpy fp64 product);
  * the worked channel example of the Jason's Study page (案例 1) and the
    planted-outlier invariant of the synthetic workloads;
  * the half-step quantization error bound against the exact product X.W;
  * round-half-to-even ties, power-of-two row scaling, row permutation.
"""
from .llm_int8 import *  # noqa: F401,F403
from .llm_int8 import __all__  # noqa: F401
