"""CPU oracle (test infrastructure only: tests, the smoke check and the benchmark's CPU baseline)."""

from .pe_oracle import *  # noqa: F401,F403
