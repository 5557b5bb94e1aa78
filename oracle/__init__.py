"""fp64 CPU oracle (test infrastructure only; see pcp_oracle's header)."""

from .pcp_oracle import *  # noqa: F401,F403
from .pcp_oracle import F, ROW_FIELDS, KIND_DECODE, KIND_HEAD, KIND_TAIL  # noqa: F401
from . import fp8  # noqa: F401,E402
