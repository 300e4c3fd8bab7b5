"""Host logic of the profile summaries (CPU only)."""
from matrix_aware_optimizer_muon_amd import profiling as P


def test_code_fingerprint_ignores_comments_only():
    real = {rel: open(f"{P.PKG}/{rel}", encoding="utf-8").read() for rel in P.KERNEL_SOURCES}
    base = P.source_hash(lambda rel: real[rel])
    assert base == P.source_hash()
    rel = "csrc/elementwise.hip"
    # comments and whitespace: same fingerprint
    edited = dict(real)
    edited[rel] = "// a new comment\n" + real[rel].replace("\n", "\n  /* note */\n", 3)
    assert P.source_hash(lambda r: edited[r]) == base
    # a code change: another fingerprint
    edited[rel] = real[rel] + "\nint unused_symbol = 1;\n"
    assert P.source_hash(lambda r: edited[r]) != base


def test_kernel_classes():
    assert P.kernel_class("void muon::gemm_dma_kernel<0, 4, 8, true>(muon::GemmParams)") == "final"
    assert P.kernel_class("void muon::gemm_kernel<0, 64, 4, false, true>(muon::GemmParams)") == "final"
    assert P.kernel_class("void muon::prep_rows_kernel<true>(muon::PrepParams, int)") == "prep"
    assert P.kernel_class("void muon::prep_tile_kernel<true, false>(muon::PrepParams, int)") == "prep"
    assert P.kernel_class("muon::write_table_kernel(muon::TableChunk, muon::MatPtrs*)") is None
