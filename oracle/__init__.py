"""fp64 CPU oracle (test infrastructure; see oracle/linear_logp.py)."""
from .linear_logp import (  # noqa: F401
    IGNORE_INDEX,
    backward,
    backward_rows,
    bf16_to_f64,
    forward,
    grad_W_rows,
    merge,
    partial,
)
