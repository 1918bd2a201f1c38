"""Host-side logic of bench.py (no GPU): the key under which the committed
counter records stay valid, the lookup of the traffic record, and the
one-GPU guard of the command line."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CSRC = os.path.join("gated_deltanet_chunked_delta_amd", "csrc")


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the library sources and the profiles under a scratch root."""
    shutil.copytree(os.path.join(ROOT, CSRC), tmp_path / CSRC)
    shutil.copytree(os.path.join(ROOT, "profiles"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _edit(path, fn):
    with open(path) as fh:
        src = fh.read()
    with open(path, "w") as fh:
        fh.write(fn(src))


def test_digest_matches_the_repository(tree):
    d = bench.kernel_sources_sha256()
    assert len(d) == 64
    bench.ROOT = ROOT
    assert bench.kernel_sources_sha256() == d


def test_digest_ignores_comments_and_blank_space(tree):
    d0 = bench.kernel_sources_sha256()
    f = tree / CSRC / "gdn_bwd.hip"
    _edit(f, lambda s: "// a new line comment\n/* and a\n block one */\n" + s.replace("\n", "\n\n", 5) + "\n   \n")
    assert bench.kernel_sources_sha256() == d0


def test_digest_changes_with_the_code(tree):
    d0 = bench.kernel_sources_sha256()
    f = tree / CSRC / "gdn_fwd.hip"
    _edit(f, lambda s: s + "\nnamespace gdn { constexpr int digest_probe = 1; }\n")
    assert bench.kernel_sources_sha256() != d0


def test_traffic_record_is_kept_only_for_unchanged_code(tree):
    rec = json.load(open(tree / "profiles" / "grad_metric_32k_traffic.json"))
    assert bench.measured_traffic("grad", "metric_32k") == rec["traffic_bytes_per_launch"]
    # the scaled figure is what the two counters say
    want = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"] + rec["write_kib_per_dispatch"] * 1024 * rec["write_scale"]
    assert abs(rec["traffic_bytes_per_launch"] - want) <= 1024
    _edit(tree / CSRC / "gdn_bwd.hip", lambda s: s.replace("min(", "min (", 1).replace("{", "{ int unused_probe = 0; (void)unused_probe;", 1))
    assert bench.measured_traffic("grad", "metric_32k") is None
    assert bench.measured_traffic("grad", "no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
