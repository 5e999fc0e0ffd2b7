"""fp64 CPU oracle (test infrastructure only; the HIP product path never imports it)."""
from .attention import *  # noqa: F401,F403
from .attention import NONE, CAUSAL, DOC_CAUSAL, all_orders  # noqa: F401
