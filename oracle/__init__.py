"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .masked_ce import (  # noqa: F401
    CEResult,
    FLCEResult,
    bf16_bits_to_f64,
    ce_masked_sum,
    ce_masked_sum_bits,
    flce,
    labelled_rows,
    logsumexp_rows,
    scale_from_count,
)
