"""Plain, slow, obviously correct CPU oracle for the binary-weight products.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
anything in this package: only the tests, the smoke check of the entry module
and the benchmark's CPU-baseline leg use it. It shares no code with the HIP
library (no kernels, headers, tables or helpers) and never reads a value the
GPU produced.

Everything is computed in fp64 with numpy. bf16 and fp16 inputs are held
exactly in fp64. Where a result has a plain definition, the function below is
that definition written out; the definitional tier (``*_loops``) spells the
sums out with ``math.fsum`` for tiny shapes.

Sources (the pages):
* "Behaviour-Relearned Quantization" (technical report page), item 02
  "Binarize experts": routed experts kept as sign bits with one scale per
  128 of them.
* "Banyan: Converting Pretrained Language Models to 1-Bit Weights with Homotopy
  On-Policy Distillation", Abstract: one sign per weight, one scale shared by a
  small group, 1.125 bits per weight, about a fourteenth of a 16-bit parent.
* "LLM binarization, Episode 01: DBF": section 1 (the representation
  W ~ D_out U D_mid V D_in and the sign convention 0 -> +1, 1 -> -1),
  section 1.1 (bit budget), section 3 (64 signs per uint64_t),
  section 4 (the deployed evaluation order and routed (token, slot) pairs).
* "BTL-4 Compact" news item: 256 experts per layer with 8 routed, router in f32.
* BWLA commentary (zhichai.net): section 3 (OKT, Kronecker orthogonal H (x) R)
  and section 5 (the same transform applied to activations).

Parity status of each function is listed in ``PINS``; every function here is
pinned by at least one test in ``tests/test_oracle_pins.py``.
"""
from .core import *  # noqa: F401,F403
from .core import PINS  # noqa: F401
