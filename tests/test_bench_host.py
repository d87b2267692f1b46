"""Host-side checks of bench.py's bookkeeping (no GPU): the HBM-traffic
summary it reports is keyed to the GEMM sources, and the key can be computed
and the committed summary parsed."""
import re

import bench


def test_gemm_source_key_is_computable():
    # every source, and the GEMM section of the shared parameter header, exists
    assert re.fullmatch(r"[0-9a-f]{64}", bench.gemm_sources_sha256())


def test_traffic_summary_parses_and_matches_row_count():
    t = bench.committed_traffic(4)
    # None only when the committed summary was taken on other GEMM sources
    assert t is None or t > 2.3e8
    assert bench.committed_traffic(5) is None  # taken at 4 rows only
