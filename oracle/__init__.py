"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .monarch_oracle import *  # noqa: F401,F403
from .monarch_oracle import __all__  # noqa: F401
