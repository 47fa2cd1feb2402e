"""CPU oracle of the sparse MoE FFN layer (test infrastructure only)."""
from .moe_oracle import *  # noqa: F401,F403
