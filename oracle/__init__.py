"""CPU oracle for the MoE route -> capacity dispatch -> expert FFN -> combine path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The GPU library never
calls it, and this package imports nothing from the GPU library.

See `oracle.moe_oracle` for what is computed and which page passage each
function follows.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
