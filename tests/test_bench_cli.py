"""CPU: bench.py's command-line contract that needs no GPU (one GPU only; asking for more exits with a message)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "no-such-layer"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "unknown workload" in (r.stderr + r.stdout)


def test_workload_by_name_or_position():
    sys.path.insert(0, ROOT)
    import bench
    import moe_workloads as W
    names = list(W.WORKLOADS)
    assert bench.pick_workload(None).name == bench.DEFAULT_WORKLOAD == "large-skewed-prefill"
    for i, n in enumerate(names):
        assert bench.pick_workload(n) is W.WORKLOADS[n]
        assert bench.pick_workload(str(i + 1)) is W.WORKLOADS[n]
    for bad in ("0", str(len(names) + 1), "mixtral"):
        try:
            bench.pick_workload(bad)
        except SystemExit as e:
            assert "unknown workload" in str(e)
        else:
            raise AssertionError(bad)


def test_cpu_baseline_runs_the_whole_batch_and_samples_experts():
    # the oracle leg on a scaled-down large skewed prefill (same tokens, experts and routing; H = 128, F = 64),
    # inputs on the host: capacity and drops are the batch's own, and the expert MLP is sampled per expert
    sys.path.insert(0, ROOT)
    import bench
    import moe_workloads as W
    cfg = W.small_config(W.workload("large-skewed-prefill"), H=128, F=64)
    inp = W.make_inputs(cfg)
    r = bench.cpu_baseline(cfg, inp, min_seconds=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0 and r["cores"] >= 1
    assert set(r["stages_s"]) == {"route", "dispatch", "expert_mlp", "combine"}
    assert r["mlp_sample"]["experts"] == 32 and r["mlp_sample"]["active_local_experts"] == 256
    assert r["oracle_seconds"] > 0
    assert "16384 tokens, capacity 512" in r["sample"]
