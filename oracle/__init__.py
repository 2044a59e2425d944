"""CPU oracle of the MoE layer forward: test infrastructure only.

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
