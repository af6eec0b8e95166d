"""fp64 CPU oracle for ring attention: test infrastructure only (see attention.py)."""
from .attention import (attention_backward, attention_forward, attention_rows, merge,  # noqa: F401
                        rank_backward, rank_forward, softmax_dot, visibility)
