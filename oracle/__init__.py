"""CPU oracle for paged MLA decode (test infrastructure; see mla_oracle.py)."""
from .mla_oracle import *  # noqa: F401,F403
