"""CPU checks of bench.py's bookkeeping: the committed HBM-traffic records still describe the
current kernel sources (bench.py reports `traffic` as null otherwise), and the algorithmic
byte and flop counts of the default workload."""

import os

import pytest

import bench
import synth

PROFILES = os.path.join(bench.ROOT, "profiles")


def _records():
    out = []
    for f in sorted(os.listdir(PROFILES)):
        if f.endswith("_hbm_traffic.md"):
            out.append(f)
    return out


@pytest.mark.parametrize("fname", _records())
def test_traffic_record_matches_current_sources(fname):
    rec = {}
    with open(os.path.join(PROFILES, fname)) as fh:
        for line in fh:
            if line.startswith("    ") and ":" in line:
                k, v = line.strip().split(":", 1)
                rec[k.strip()] = v.strip()
    stage, config = rec["stage"], rec["workload"]
    spec = synth.spec_for(config)
    matches = [key for key in bench.KERNEL_SOURCES
               if key[1] == spec.weight and key[2] == stage
               and fname == f"{bench.KERNEL_SOURCES[key][0].rsplit('.', 1)[0]}_{stage}_{config}_hbm_traffic.md"]
    assert len(matches) == 1, f"{fname}: no kernel source entry"
    name, digest = bench.kernel_digest(*matches[0])
    assert rec["kernel_source_sha256"] == digest, f"{fname} was measured on other sources; measure it again"
    assert bench.recorded_traffic(name, stage, config, digest) == float(rec["traffic_bytes_per_launch"])


def test_default_workload_is_the_largest_single_gpu_layer():
    assert bench.WORKLOADS["dsv3_prefill_bf16"].startswith("DeepSeek-V3-shaped bf16 prefill")
    spec = synth.spec_for("dsv3_prefill_bf16")
    flops, byts = bench.algorithmic(spec, 187, "gate_up")
    assert flops == 4.0 * 65536 * 7168 * 2048                      # 3.85 TFLOP
    assert byts == 187 * 2 * 2048 * 7168 * 2 + 8192 * 7168 * 2       # weights + x; not `a`
    assert bench.intermediate_bytes(spec, "gate_up") == 65536 * 2048 * 2


def test_fp8_algorithmic_counts():
    spec = synth.spec_for("dsv3_fp8_f32scale")
    _, byts = bench.algorithmic(spec, 157, "gate_up")
    # e4m3 weights + one float32 scale per 128x128 block, x codes + their row scales
    assert byts == 157 * 2 * 2048 * 7168 * (1 + 4 / 16384) + 4096 * 7168 + 4096 * 56 * 4
    assert bench.intermediate_bytes(spec, "down") == 32768 * 2048 + 32768 * 16 * 4


def test_qwen_prefill_algorithmic_counts():
    spec = synth.spec_for("qwen_prefill_bf16")
    flops, byts = bench.algorithmic(spec, 60, "gate_up")
    assert flops == 4.0 * 16384 * 2048 * 1408                      # 189.0 GFLOP
    assert byts == 60 * 2 * 1408 * 2048 * 2 + 4096 * 2048 * 2      # 709.0 MB
    df, db = bench.algorithmic(spec, 60, "down")
    assert df == 2.0 * 16384 * 2048 * 1408
    assert db == 60 * 1408 * 2048 * 2 + 4096 * 2048 * 2             # W_down + out
    lf, lb = bench.layer_totals(spec, 60)
    assert lf == 6.0 * 16384 * 2048 * 1408
    assert lb == 60 * 3 * 1408 * 2048 * 2 + 2 * 4096 * 2048 * 2 + 8 * 16384


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=bench.ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line
