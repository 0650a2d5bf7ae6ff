"""Host-side checks of bench.py: the one-GPU contract and the CPU-oracle leg
(no GPU involved)."""
import json

import bench


def _last_json(text: str) -> dict:
    lines = [ln for ln in text.strip().splitlines() if ln.startswith("{")]
    assert lines, text
    return json.loads(lines[-1])


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    out = _last_json(capsys.readouterr().out)
    assert "error" in out and "one GPU" in out["error"]


def test_whole_oracle_on_the_tiny_workload(capsys):
    assert bench.main(["--cpu-full", "tiny", "--cpu-threads", "1"]) == 0
    out = _last_json(capsys.readouterr().out)
    assert out["cpu_full"] == "tiny" and out["kind"] == "oracle" and out["cores"] == 1
    assert out["total_s"] >= out["forward_s"] >= 0 and out["backward_s"] is None
    assert out["executed_fwd_tflop"] > 0 and out["cpu_model"]


def test_source_hash_is_stable_and_content_based(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("x")
    h1 = bench.source_hash([str(a)])
    assert h1 == bench.source_hash([str(a)])
    a.write_text("y")
    assert bench.source_hash([str(a)]) != h1
