"""fp64 CPU oracle for the FLARE++ mixer forward pass, its gradients and
its front end (input projections and head-wise normalisation).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in
__graft_entry__ and by the CPU-baseline leg of bench.py, never by the GPU
library or its Python binding.
"""
from .flarepp_oracle import *  # noqa: F401,F403
from .flarepp_backward import *  # noqa: F401,F403
from .flarepp_oracle import __all__ as _fwd_all
from .flarepp_backward import __all__ as _bwd_all
from .flarepp_frontend import *  # noqa: F401,F403
from .flarepp_frontend import __all__ as _fe_all

__all__ = list(_fwd_all) + list(_bwd_all) + list(_fe_all)
