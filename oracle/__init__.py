"""fp64 CPU oracle: test infrastructure only (see attention.py and fir.py)."""
from .attention import (attention_backward, attention_forward, attention_rows, merge,  # noqa: F401
                        rank_backward, rank_forward, softmax_dot, visibility)
from .fir import fir_forward, fir_shards  # noqa: F401
