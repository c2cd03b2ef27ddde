"""fp64 CPU oracle (test infrastructure only; never imported by the product path)."""
from .monarch_oracle import *  # noqa: F401,F403
from .monarch_oracle import __all__ as _fwd_all
from .monarch_backward import *  # noqa: F401,F403
from .monarch_backward import __all__ as _bwd_all
from .monarch_refine import *  # noqa: F401,F403
from .monarch_refine import __all__ as _ref_all

__all__ = list(_fwd_all) + list(_bwd_all) + list(_ref_all)
