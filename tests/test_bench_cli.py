"""The benchmark's command line on the CPU: it measures one GPU only and says
so (before touching a GPU) when asked for more."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_unknown_workload_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "no_such_layer"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_per_unit():
    # prepare: 2 bytes read, 0.5 + 0.5 code bytes, 2/32 scale bytes and 1/8 mask byte written per element;
    # two-path GEMM: both activation operands and the weight at 17/32 byte per element, fp32 Y
    b = _bench_module()
    assert b.prepare_bytes(2048, 14336) == 2048 * 14336 * 3.1875
    assert b.prepare_bytes(1, 4096, gamma=True) == 4096 * 3.1875 + 2 * 4096
    assert b.gemm_bytes(1, 8192, 28672) == 2 * 28672 * 17 / 32 + 8192 * 28672 * 17 / 32 + 4 * 8192
    alg, exe = b.gemm_flops(2048, 28672, 4096)
    assert alg == 3.0 * 2048 * 28672 * 4096 and exe == 4.0 * 2048 * 28672 * 4096


def test_recorded_traffic_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    # a counter record carries the SHA-256 of the kernel sources; a record taken on other sources reads as None
    import json
    b = _bench_module()
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = b.source_digest("gemm_down")
    (prof / "traffic.json").write_text(json.dumps({
        "w/gemm_down": {"hbm_bytes_per_launch": 123, "source_sha256": digest},
        "w/gemm_stale": {"hbm_bytes_per_launch": 456, "source_sha256": "0" * 64}}))
    real_join = os.path.join
    monkeypatch.setattr(b.os.path, "join",
                        lambda *p: str(prof / "traffic.json") if p[-1] == "traffic.json" else real_join(*p))
    assert b.recorded_traffic("w", "gemm_down") == 123
    assert b.recorded_traffic("w", "gemm_stale") is None
    assert b.recorded_traffic("w", "absent") is None


def test_traffic_records_are_well_formed():
    import json
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    assert recs
    for key, r in recs.items():
        workload, stage = key.split("/")
        assert workload and stage
        assert len(r["source_sha256"]) == 64
        # bytes per launch = calibrated FETCH_SIZE + WRITE_SIZE (KiB)
        want = (r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"]) * 1024
        assert abs(r["hbm_bytes_per_launch"] - want) <= 1024, key
