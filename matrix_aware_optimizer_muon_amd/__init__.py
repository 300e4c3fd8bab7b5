"""MI355X-native Muon optimizer step (Gram-space Newton-Schulz, periodic
RowNorm) behind a C ABI (include/muon.h, libmuon.so)."""
from ._lib import Plan, MuonError, default_hparams, load  # noqa: F401
