"""CPU oracle for sparse causal flash attention -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The HIP product path never imports, links or runs it.
"""
from .scfa_oracle import *  # noqa: F401,F403
from .scfa_oracle import Q_PAD, K_PAD  # noqa: F401
