"""CPU oracle for the QLoRA NF4 linear layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here.
"""
from .nf4_oracle import *  # noqa: F401,F403
