"""CPU oracle -- test infrastructure only (see ``kos_oracle``)."""
from .kos_oracle import *  # noqa: F401,F403
