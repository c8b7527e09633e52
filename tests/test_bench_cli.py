"""bench.py's command-line contract on the CPU: more than one GPU is
refused with a message and a nonzero exit status before any GPU is touched
(the build runs on one GPU; the PCP rank share is its own workload)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]


def _fake_smi(tmp_path, body):
    tool = tmp_path / "amd-smi"
    tool.write_text("#!/bin/sh\ncat <<'JSON'\n" + body + "\nJSON\n")
    tool.chmod(0o755)
    return str(tmp_path)


def test_power_sample_parses_amd_smi_json(tmp_path, monkeypatch):
    # one reading as amd-smi prints it for GPU 0: socket power and a clock
    # per XCD; the sampler returns the power and the XCDs' mean clock
    clocks = {f"gfx_{i}": {"clk": {"value": 1600 + 10 * i, "unit": "MHz"}, "max_clk": {"value": 2400}}
              for i in range(8)}
    body = json.dumps([{"gpu": 0, "power": {"socket_power": {"value": 1389, "unit": "W"}, "gfx_voltage": "N/A"},
                        "clock": dict(clocks, mem_0={"clk": {"value": 1900}})}])
    monkeypatch.setenv("PATH", _fake_smi(tmp_path, body) + os.pathsep + os.environ["PATH"])
    sys.path.insert(0, ROOT)
    import bench
    watts, mhz = bench._smi_sample()
    assert watts == 1389.0
    assert mhz == sum(1600 + 10 * i for i in range(8)) / 8


def test_power_sample_without_a_reading(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setenv("PATH", _fake_smi(tmp_path, "not json") + os.pathsep + os.environ["PATH"])
    assert bench._smi_sample() is None
    monkeypatch.setenv("PATH", str(tmp_path / "nowhere"))
    assert bench._smi_sample() is None
