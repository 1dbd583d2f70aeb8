"""Host-side checks of bench.py's contract (no GPU).

Only one GPU is measured: asking for more must fail with a message before
any device work. The HBM-traffic figure reported beside the roofline must
come from a counter record whose source hash matches the decode sources.
"""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_counted_traffic_follows_the_sources(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    name = "hybrid_global_traffic.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        import pytest
        pytest.skip("no counter record committed yet")
    rec = json.load(open(path))
    # the committed record matches the committed sources
    assert bench.counted_traffic(name) == rec["traffic_bytes_per_launch"]
    # a record taken on other sources is not reported
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    for f in rec["source_files"]:
        dst = fake / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        dst.write_bytes(open(os.path.join(ROOT, f), "rb").read() + b"\n// changed\n")
    (fake / "profiles" / name).write_text(json.dumps(rec))
    monkeypatch.setattr(bench.os.path, "abspath", lambda p: str(fake / "bench.py"))
    assert bench.counted_traffic(name) is None


def test_every_only_choice_selects_a_workload():
    """Each `--only` value names the headline, its global layer or one extra."""
    import bench
    ap_choices = None
    for a in bench.build_parser()._actions if hasattr(bench, "build_parser") else []:
        if a.dest == "only":
            ap_choices = a.choices
    if ap_choices is None:
        import re
        src = open(bench.__file__).read()
        ap_choices = re.findall(r'"([a-z_0-9]+)"', src[src.index('"--only", choices=['):src.index('default=None, help="time a single')])
    extras = {bench.ONLY_KEY.get(n, n) for n in bench.EXTRA_NAMES}
    for c in ap_choices:
        assert c in extras or c in ("hybrid", "hybrid_global"), c
    assert extras <= set(ap_choices)
