"""The committed traffic profile belongs to the committed GEMM kernels.

bench.py reports the headline GEMM's HBM traffic from profiles/traffic_<workload>.json only while
that file's sha256 of the GEMM sources matches the sources in the tree (otherwise the line's
`traffic` is null). This test fails when a GEMM source changes without the counters being taken
again, so the committed profile never describes other code than the committed kernels.
"""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_profile_matches_the_gemm_sources():
    path = os.path.join(ROOT, "profiles", f"traffic_{bench.HEADLINE}.json")
    rec = json.load(open(path))
    assert rec["gemm_source_sha256"] == bench.gemm_source_digest()
    assert rec["workload"] == bench.HEADLINE and rec["weights"] == "packed"
    for stage in ("expert_gemm1_gelu", "expert_gemm2"):
        assert rec["bytes_per_launch"][stage] > 0


def test_traffic_profile_is_read_back_by_the_bench():
    path = os.path.join(ROOT, "profiles", f"traffic_{bench.HEADLINE}.json")
    assert bench.stored_traffic(path, "expert_gemm1_gelu", "packed") is not None
    assert bench.stored_traffic(path, "expert_gemm1_gelu", "row-major") is None
