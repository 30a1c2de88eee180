"""CPU oracle (test infrastructure only; never used by the product path)."""
from .ref import (GROUP, QMAX, TOL, dequant, linear_ref, linear_rows, lowrank_term, pack,  # noqa: F401
                  quantize_layer, quantize_rtn, rel_err_inf, sparse_term,
                  split_outliers, unpack)
