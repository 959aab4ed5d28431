"""fp64 CPU oracle for attention (test infrastructure; never used by the HIP path)."""
from .attention import (  # noqa: F401
    backward,
    forward,
    head_backward,
    head_forward,
    head_blocked,
    visible,
)
