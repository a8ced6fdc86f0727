"""bench.py's host-side contract, without a GPU: a request for more than one GPU
exits with a message before touching a device, the kernel-code digest that keys
the committed counter records ignores comments but not code, and the default
stream schedule follows the number of groups and the placement of appends."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_first_group_needs_a_group_count_in_range():
    """--first-group picks groups G0.. of a workload: refused (before any device call)
    without --groups or with G0 outside the workload's groups."""
    for extra in (["--first-group", "6"], ["--groups", "6", "--first-group", "24"],
                  ["--groups", "2", "--first-group", "2"]):
        wl = "evict_r256_128k_g2" if extra[-1] == "2" else "r64_64k128k_g24x3"
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", wl] + extra,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2, extra
        assert "--first-group" in r.stderr and r.stdout == ""


def test_code_digest_ignores_comments_only(tmp_path):
    import bench
    base = "int f(int a) {\n  return a + 1;  // one more\n}\n/* block\n   comment */\n"
    same = "// header\nint f(int a) {\n    return a + 1;\n}\n"
    other = "int f(int a) {\n  return a + 2;\n}\n"
    paths = []
    for i, text in enumerate((base, same, other)):
        p = tmp_path / f"k{i}.hip"
        p.write_text(text)
        paths.append(str(p))
    d = [bench.code_digest(p) for p in paths]
    assert d[0] == d[1]
    assert d[0] != d[2]


def test_traffic_record_needs_matching_code(tmp_path, monkeypatch):
    """A counter record is reported only for the kernel code it was taken on."""
    import json
    import bench
    prof = tmp_path / "profiles"
    csrc = tmp_path / "serving_pb_lru_amd" / "csrc"
    prof.mkdir()
    csrc.mkdir(parents=True)
    (csrc / "k_gather.hip").write_text("int g() { return 1; }\n")
    rec = {"k_gather_hip_code_sha256": bench.code_digest(str(csrc / "k_gather.hip")),
           "traffic_bytes_per_launch": 12345}
    (prof / "traffic_k_gather_w_split.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.gather_traffic("w", "split") == 12345
    assert bench.gather_traffic("w", "layer") is None            # no record for that form
    (csrc / "k_gather.hip").write_text("// note\nint g() { return 1; }\n")
    assert bench.gather_traffic("w", "split") == 12345           # a comment changes nothing
    (csrc / "k_gather.hip").write_text("int g() { return 2; }\n")
    assert bench.gather_traffic("w", "split") is None            # the code changed


def test_auto_stream_schedule():
    """--streams auto: a gather stream beside one step stream (one group), a stream
    per group (two) or two alternating step streams (more); no gather stream under
    the second placement of appends; an explicit schedule is kept."""
    import bench
    assert bench.schedule_for(1, "lowest") == "one+gather"
    assert bench.schedule_for(2, "lowest") == "group+gather"
    assert bench.schedule_for(4, "lowest") == "two+gather"
    assert bench.schedule_for(24, "lowest") == "two+gather"
    assert bench.schedule_for(1, "ring") == "one"
    assert bench.schedule_for(2, "ring") == "group"
    assert bench.schedule_for(4, "ring") == "two"
    assert bench.schedule_for(4, "lowest", "group") == "group"
