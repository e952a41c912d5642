"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .xattn_oracle import *  # noqa: F401,F403
from .xattn_oracle import __all__  # noqa: F401
