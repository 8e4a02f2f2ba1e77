"""Host logic of bench.py (no GPU): the counter-traffic lookup reads the committed
rocprofv3 summaries by section and refuses them for other kernel sources."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_traffic_sections_parse_and_are_tied_to_sources():
    cases = [
        ("gqa_decode_kernel.hbm-counters.decode-64seq.txt", bench.DECODE_SOURCES, None),
        ("gqa_prefill_kernel.suffix-prefill-8x142000+2048.txt", bench.PREFILL_SOURCES, "gqa_prefill_kernel"),
        ("mla_kernel.mla-mtp3-decode-64seq-ctx32k-256k.txt", bench.MLA_SOURCES, "mla_kernel<false"),
        (bench.SPARSE_PROFILE, bench.INDEXER_SOURCES, "indexer_kernel<4> (FP8 keys)"),
        (bench.SPARSE_PROFILE, bench.INDEXER_SOURCES, "indexer_kernel<4> (MXFP4 keys, packed layout)"),
        (bench.SPARSE_PROFILE, bench.TOPK_SOURCES, "topk_kernel (FP8 keys run)"),
        (bench.SPARSE_PROFILE, bench.MLA_SOURCES, "mla_kernel<true, 2, 4, true> (sparse, FP8 keys run)"),
    ]
    for fname, sources, section in cases:
        path = os.path.join(ROOT, "profiles", fname)
        text = open(path).read()
        assert "source_sha256" in text and "traffic_bytes_per_launch" in text, fname
        # another source list never matches the stamp
        other = [s for s in bench.DECODE_SOURCES + bench.TOPK_SOURCES if s not in sources][:1] + sources
        assert bench.measured_traffic(fname, other, section=section) is None, (fname, section)
        # a section that does not exist yields nothing
        assert bench.measured_traffic(fname, sources, section="no such kernel") is None, fname


def test_traffic_values_are_plausible_when_current():
    """When the stamp matches the sources, the traffic is the summary's number: a positive
    byte count at least the kernel's algorithmic bytes for the HBM-bound kernels."""
    t = bench.measured_traffic("gqa_decode_kernel.hbm-counters.decode-64seq.txt", bench.DECODE_SOURCES)
    if t is not None:
        assert t >= 2190147584
    t = bench.measured_traffic(bench.SPARSE_PROFILE, bench.TOPK_SOURCES, section="topk_kernel (FP8 keys run)")
    if t is not None:
        assert t >= 2214600704
