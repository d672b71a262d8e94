"""Host logic of bench.py (no GPU): byte accounting of the metric and the
roofline, the source-hash gate on the committed counter profile, the SQNR
helper and the one-GPU guard."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

M, N, K = 32, 4096, 3072
X_BYTES, Y_BYTES, BIAS_BYTES = M * K * 2, M * N * 2, N * 2

# Packed weight + scale bytes of nn.Linear(3072 -> 4096), written out per format:
# two E2M1/INT4 codes per byte, one E4M3 code per byte; INT4 bf16 scale per 128 K,
# FP8 fp32 scale per row, NVFP4 E4M3 per 16 K + fp32 global, MXFP4 E8M0 per 32 K.
EFFECTIVE = {
    "int4": N * K // 2 + N * (K // 128) * 2,
    "fp8": N * K + N * 4,
    "nvfp4": N * K // 2 + N * (K // 16) + 4,
    "mxfp4": N * K // 2 + N * (K // 32),
    "static_fp8": N * K + N * 4 + 4,
}


@pytest.mark.parametrize("name", sorted(EFFECTIVE))
def test_effective_bytes(name):
    assert bench.effective_bytes(name) == EFFECTIVE[name]


def test_algorithmic_bytes():
    for fmt in ("int4", "fp8", "nvfp4", "mxfp4"):
        assert bench.algorithmic_bytes(fmt) == EFFECTIVE[fmt] + X_BYTES + BIAS_BYTES + Y_BYTES
    assert bench.algorithmic_bytes("int4") == 6_955_008
    assert bench.algorithmic_bytes("fp8") == 13_066_240
    assert bench.algorithmic_bytes("nvfp4") == 7_544_836
    assert bench.algorithmic_bytes("mxfp4") == 7_151_616
    # static GEMM: E4M3 X in, no bias; act Q: bf16 X in, E4M3 X out, the scale
    assert bench.algorithmic_bytes("static_gemm") == EFFECTIVE["static_fp8"] + M * K + Y_BYTES == 12_959_748
    assert bench.algorithmic_bytes("static_q") == X_BYTES + M * K + 4 == 294_916


def _profile(tmp_path, sha):
    rec = {"src_sha256": sha, "calibration": {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0},
           "bytes_per_launch": {"fp8": 14_500_000}}
    p = tmp_path / "counters.md"
    p.write_text("# counters\n\n<!-- traffic %s -->\n" % json.dumps(rec))
    return str(p)


def test_traffic_only_for_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "COUNTERS_PROFILE", _profile(tmp_path, bench.kernel_source_hash()))
    assert bench.committed_traffic() == {"fp8": 14_500_000}
    monkeypatch.setattr(bench, "COUNTERS_PROFILE", _profile(tmp_path, "0" * 16))
    assert bench.committed_traffic() == {}
    monkeypatch.setattr(bench, "COUNTERS_PROFILE", str(tmp_path / "missing.md"))
    assert bench.committed_traffic() == {}


def test_committed_profile_parses():
    text = open(bench.COUNTERS_PROFILE).read()
    assert "<!-- traffic " in text
    assert "rocprofv3" in text  # the command that produced it is recorded


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_sqnr_db_closed_forms():
    """The SQNR the bench reports: a uniform relative error e gives -20 log10(e)
    dB; identical outputs give infinity; bf16 inputs are widened exactly."""
    import torch

    ref = torch.full((4, 8), 3.0, dtype=torch.bfloat16)
    y = ref * (1 + 2.0 ** -6)  # 3 * (1 + 1/64) is exact in bf16
    assert bench.sqnr_db(ref, y) == pytest.approx(-20 * math.log10(2.0 ** -6), abs=0.01)
    assert bench.sqnr_db(ref, ref.clone()) == float("inf")
    # a sign flip of half the elements: error power 4x half the signal -> -3.01 dB
    z = ref.clone()
    z[:2] = -z[:2]
    assert bench.sqnr_db(ref, z) == pytest.approx(-10 * math.log10(2.0), abs=0.01)
