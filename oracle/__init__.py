"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .flce_oracle import (FILTER_EPS_DEFAULT, IGNORE_INDEX_DEFAULT, dH_rows, dW_rows,
                          filter_block_stats, linear_cross_entropy, lse_all, row_scale,
                          valid_rows)

__all__ = ["linear_cross_entropy", "lse_all", "dH_rows", "dW_rows", "row_scale", "valid_rows",
           "filter_block_stats", "FILTER_EPS_DEFAULT", "IGNORE_INDEX_DEFAULT"]
