"""Host-side checks of bench.py's contract (no GPU): the refusal of more than
one GPU, the algorithmic byte and operation counts behind `roofline`, and the
guard that drops a counter-derived traffic figure taken on another kernel
source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as WL  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


# Rotate+quantise algorithmic bytes per launch (bf16 input, codes at their
# packed width, a float32 scale per token, the float32 mean when centred;
# MXFP4: E2M1 codes and one E8M0 byte per 32), the figures of the workload
# table the roofline is quoted against.
@pytest.mark.parametrize("cid,nbytes", [(1, 787_456), (2, 31_473_664), (3, 23_609_344), (4, 31_490_048),
                                        (5, 85_196_800)])
def test_rotate_quant_algorithmic_bytes(cid, nbytes):
    s = WL.config_spec(cid)
    assert bench._act_bytes(s, s.M, s.K) == nbytes


# 2 M K N integer operations per linear.
@pytest.mark.parametrize("cid,N,gops", [(1, 1024, 0.537), (2, 3072, 77.31), (2, 12288, 309.24), (3, 1920, 30.20),
                                        (3, 7680, 120.80), (5, 14336, 962.07)])
def test_gemm_operation_counts(cid, N, gops):
    s = WL.config_spec(cid)
    assert N in s.Ns
    assert round(2.0 * s.M * s.K * N / 1e9, 2 if gops > 1 else 3) == gops


def test_traffic_needs_the_current_source(tmp_path):
    src = "k_gemm_fp6.hip"
    good = {"source_sha1": bench._src_hash([src]), "hbm_bytes_per_launch": 12345}
    (tmp_path / "good.json").write_text(json.dumps(good))
    (tmp_path / "stale.json").write_text(json.dumps({**good, "source_sha1": "0" * 16}))
    (tmp_path / "broken.json").write_text("{")
    d = str(tmp_path)
    assert bench._traffic("good.json", [src], d) == 12345
    assert bench._traffic("stale.json", [src], d) is None
    assert bench._traffic("broken.json", [src], d) is None
    assert bench._traffic("missing.json", [src], d) is None
