"""Oracle of the top-2 MoE FFN layer -- test infrastructure only (see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
