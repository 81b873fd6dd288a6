"""Float64 CPU oracle (test infrastructure only; see gptq_oracle's header)."""
from .gptq_oracle import *  # noqa: F401,F403
from .gptq_oracle import NotPositiveDefinite, layer_objective_per_channel  # noqa: F401
