"""CPU oracle (test infrastructure only; never used by the product path)."""
from .ref import (GROUP, QMAX, TOL, dequant, dequant_gidx, linear_ref, linear_ref_gidx,  # noqa: F401
                  linear_rows, linear_w4a8_ref, lowrank_term, pack, pack3, quantize_act_int8, quantize_layer,
                  quantize_rtn, quantize_rtn_gidx, rel_err_inf, sparse_term, split_outliers, unpack, unpack3)
