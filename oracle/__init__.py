"""fp64 CPU oracle for MLA -- test infrastructure only (see mla_oracle's header)."""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import __all__  # noqa: F401
