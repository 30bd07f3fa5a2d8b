"""CPU oracle of the HiLS forward pass (test infrastructure only; see hils_oracle)."""
from .hils_oracle import *  # noqa: F401,F403
