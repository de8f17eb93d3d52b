"""CPU oracle of the KV-cache refinement decode step.  TEST INFRASTRUCTURE ONLY:
imported by tests/, the smoke check and the benchmark's CPU-baseline leg, never
by the product path."""
from .kv_oracle import *  # noqa: F401,F403
