"""CPU oracle (test infrastructure only; see dcoco_oracle's header)."""
from .dcoco_oracle import *  # noqa: F401,F403
from . import dcoco_oracle  # noqa: F401
