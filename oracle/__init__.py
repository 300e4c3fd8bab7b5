"""CPU float64 oracle for the Muon and periodic-RowNorm steps.

Test infrastructure only: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the product path."""
from .muon_oracle import *  # noqa: F401,F403
