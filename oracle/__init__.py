"""CPU oracle of the routed MoE layer (test infrastructure; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
