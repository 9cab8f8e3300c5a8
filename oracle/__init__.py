"""Oracle for the dropless MoE layer: test infrastructure only (see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
