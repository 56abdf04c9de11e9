"""CPU oracle for the INT8 KV-cache path (test infrastructure only)."""
from .kvq_oracle import *  # noqa: F401,F403
