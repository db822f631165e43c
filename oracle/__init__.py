"""fp64 CPU oracle for the W4A16 int4 weight-only linear layer.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  The product package
(w4a16_int4_weight_linear_amd) never imports it and it never imports the
product: the two share no code, headers, tables or helpers.  Inputs for both
come from the ``synth`` generators, which hold none of the layer's arithmetic.

Every function is pinned by the CPU tests (tests/test_oracle_pins.py) to facts
fixed by the scheme and by mathematics (hand-derived words and codes in
tests/golden/, closed forms, exact integer arithmetic, invariants, brute-force
loops).  No function here is left "parity unpinned".
"""

from .reference import (GROUPS, quantize, pack, unpack, dequantize, linear, linear_rows,
                        linear_cols, linear_loops, grouped_linear, silu, swiglu_linear, moe_route,
                        moe_combine, moe_layer, grouped_swiglu_linear, moe_ffn)
from .check import compare, Report, ELEM_TOL, ROW_TOL

__all__ = ["GROUPS", "quantize", "pack", "unpack", "dequantize", "linear", "linear_rows",
           "linear_cols", "linear_loops", "grouped_linear", "silu", "swiglu_linear", "moe_route", "moe_combine", "moe_layer",
           "grouped_swiglu_linear", "moe_ffn",
           "compare", "Report",
           "ELEM_TOL", "ROW_TOL"]
