"""Host-side logic of bench.py (no GPU): the per-step algorithmic byte model and the one-GPU
guard. The byte figures are the per-step totals of the decode workloads' shapes worked out by
hand (indexer keys, q, head weights, the score round trip, indices twice, absorbed q, the
selected 576-wide rows and the fp32 output), plus the fp32 log-sum-exp per (query, head)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402

# workload -> step bytes without the log-sum-exp output
HAND_WORKED = {
    "tiny_fp32_decode_256": 317_968,
    "glm_decode_b1_8k": 4_751_488,
    "batched_decode_b32_32k": 359_665_664,
    "long_decode_b8_128k": 297_534_464,
}


@pytest.mark.parametrize("name", sorted(HAND_WORKED))
def test_step_bytes(name):
    wl = workloads.WORKLOADS[name]
    b = bench.algorithmic_bytes(wl)
    lse = wl.B * wl.n_q * wl.Hm * 4
    assert b["step"] - lse == HAND_WORKED[name]
    # the step is the three calls with each intermediate counted once as a write and once as a read
    assert b["step"] == b["index_score"] + b["topk"] + b["sparse_mla"]


def test_batched_decode_key_stream():
    wl = workloads.WORKLOADS["batched_decode_b32_32k"]
    # 32 sequences x 32768 keys x 128 bf16 = 268 MB of keys, plus q, w and 4.2 MB of scores
    assert bench.algorithmic_bytes(wl)["index_score"] == 32 * 32768 * 128 * 2 + 32 * 32 * 128 * 2 \
        + 32 * 32 * 4 + 32 * 32768 * 4


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True,
                       text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_runs_in_processes():
    """The oracle baseline forks worker processes over independent sequences and reports the
    processes it used (a short run on the tiny workload)."""
    wl = workloads.WORKLOADS["tiny_fp32_decode_256"]
    inp = workloads.gen_all(wl, 0)
    r = bench.cpu_baseline(wl, inp, seconds_target=0.3, workers=2)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert "2 processes" in r["sample"]
