"""CPU oracle (test infrastructure only; see wamc_oracle's header)."""
from . import wamc_oracle  # noqa: F401
