"""fp64 CPU oracle for tiled exact attention.  Test infrastructure only: the
product path never imports it (see attention.py's header)."""

from .attention import (visibility, head_forward, head_backward, head_probabilities,
                        head_rows, forward, backward, visibility_kv, head_forward_kv,
                        forward_kv, forward_varlen)

__all__ = ["visibility", "head_forward", "head_backward", "head_probabilities",
           "head_rows", "forward", "backward", "visibility_kv", "head_forward_kv",
           "forward_kv", "forward_varlen"]
