"""CPU oracle (test infrastructure only; never used on the product path)."""
from .oracle import *  # noqa: F401,F403
