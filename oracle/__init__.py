"""fp64 CPU oracle: test infrastructure only (see attention.py and fir.py)."""
from .attention import (attention_backward, attention_backward_rows, attention_forward,  # noqa: F401
                        attention_rows, merge, rank_backward, rank_forward, softmax_dot,
                        visibility)
from .fir import fir_forward, fir_shards  # noqa: F401
