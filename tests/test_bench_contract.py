"""The benchmark's host-side contract without a GPU: argument defaults, the
one-GPU refusal, the roofline bound chosen from algorithmic intensity, and the
traffic lookup keyed by the kernel sources."""
import json

import pytest

import bench
from gqa_decode_attention_fr_amd import workloads as W


def test_defaults_and_one_gpu_only(capsys):
    a = bench.parse_args([])
    assert (a.gpus, a.steps, a.warmup) == (1, 200, 20)
    assert a.workload == W.PI05_ACTION_STEP.name
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("w,bound", [(W.PI05_ACTION_STEP, "hbm"), (W.CAUSAL_TAIL, "hbm"),
                                     (W.LONG_CONTEXT, "mfma"), (W.PREFILL_PI05, "mfma"),
                                     (W.GQA_KV8, "hbm")])
def test_roofline_bound_follows_intensity(w, bound):
    r = bench.roofline(w, kern_ms=0.01, achieved_gbs=1000.0, traffic=None)
    assert r["bound"] == bound
    if bound == "hbm":
        assert (r["unit"], r["peak"]) == ("GB/s", 8000.0) and r["frac"] == 0.125
    else:
        tflops = w.flops() / 1e-5 / 1e12
        assert r["unit"] == "TFLOP/s" and abs(r["achieved"] - round(tflops, 2)) < 1e-9


def test_traffic_only_for_the_current_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    rec = {"variant": 1, "hbm_bytes_per_launch": 12345}
    f.write_text(json.dumps({"kernel_hash": bench.kernel_hash(),
                             "workloads": {W.PI05_ACTION_STEP.name: rec}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for(W.PI05_ACTION_STEP.name, 1) == 12345
    assert bench.traffic_for(W.PI05_ACTION_STEP.name, 2) is None      # other variant
    assert bench.traffic_for(W.TINY.name, 1) is None                  # not measured
    f.write_text(json.dumps({"kernel_hash": "stale", "workloads": {W.PI05_ACTION_STEP.name: rec}}))
    assert bench.traffic_for(W.PI05_ACTION_STEP.name, 1) is None      # sources changed


def test_committed_traffic_is_well_formed():
    """profiles/traffic.json holds calibrated counters; when it was taken on the
    kernel sources in the tree, bench.py reports its figure (else null)."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    cal = t["calibration"]
    assert 0.3 < cal["fetch_factor"] < 3 and 0.3 < cal["write_factor"] < 3
    if t["kernel_hash"] != bench.kernel_hash():
        pytest.skip("counters taken on other kernel sources: bench.py reports traffic null")
    assert bench.traffic_for(W.PI05_ACTION_STEP.name, 1) > W.PI05_ACTION_STEP.algorithmic_bytes()


def test_committed_traffic_covers_every_workload():
    """Each line `bench.py --workload all` prints has counter traffic of its own
    main kernel, at least its algorithmic bytes less the calibration's slack."""
    with open(bench.TRAFFIC_FILE) as fh:
        t = json.load(fh)
    if t["kernel_hash"] != bench.kernel_hash():
        pytest.skip("counters taken on other kernel sources: bench.py reports traffic null")
    for w in W.WORKLOADS + W.EXTRA_WORKLOADS:
        tr = bench.traffic_for(w.name, 1)
        assert tr is not None and tr > 0.95 * w.algorithmic_bytes(), w.name
    for name in (bench.COPY_WORKLOAD, bench.QKV_WORKLOAD):
        rec = t["workloads"][name]
        assert bench.traffic_for(name) == rec["hbm_bytes_per_launch"]
        assert rec["hbm_bytes_per_launch"] > 0.95 * rec["algorithmic_bytes_per_launch"]
