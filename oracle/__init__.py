"""CPU oracle (test infrastructure only; see lora_oracle.py)."""
from .lora_oracle import *  # noqa: F401,F403
