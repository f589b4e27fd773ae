"""fp64 CPU oracle (test infrastructure only; see attn_fp64.py)."""
from .attn_fp64 import *  # noqa: F401,F403
