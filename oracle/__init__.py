"""CPU oracle of the MoE FFN forward (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
