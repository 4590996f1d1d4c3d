"""Float64 CPU oracle (test infrastructure only; see hyena_oracle)."""
from .hyena_oracle import *  # noqa: F401,F403
from .hyena_oracle import __all__  # noqa: F401
