"""CPU oracle for paged KV attention (test infrastructure only; see pa_oracle)."""
from .pa_oracle import *  # noqa: F401,F403
