"""Host-side logic of bench.py: no GPU needed.

- the counter summaries in profiles/ are tied to the decode code they were
  taken on by a hash of its non-comment lines, and roofline.traffic is read
  from them only while that code is unchanged;
- more than one GPU is refused with a message and exit status 2.
"""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SOURCE = """// header comment
int f(int x) {   // trailing comment
    return x + 1;
}
"""


def write(path, text):
    with open(path, "w") as f:
        f.write(text)


def test_code_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "decode.hip"
    write(src, SOURCE)
    monkeypatch.setattr(bench, "DECODE_SRC", str(src))
    h0 = bench.decode_code_sha256()
    write(src, "// another header\n\n" + SOURCE.replace("trailing comment", "reworded"))
    assert bench.decode_code_sha256() == h0
    write(src, SOURCE.replace("x + 1", "x + 2"))
    assert bench.decode_code_sha256() != h0


def test_traffic_read_only_for_the_profiled_code(tmp_path, monkeypatch):
    src = tmp_path / "decode.hip"
    write(src, SOURCE)
    monkeypatch.setattr(bench, "DECODE_SRC", str(src))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_profile("mixed") is None          # no summary
    summary = ("| x | y |\n\ndecode_code_sha256: %s\ntraffic_bytes_per_launch: 1.729077e+09\n"
               % bench.decode_code_sha256())
    write(tmp_path / "decode_mixed_traffic.md", summary)
    assert bench.traffic_from_profile("mixed") == pytest.approx(1.729077e9)
    write(src, SOURCE.replace("x + 1", "x - 1"))                 # the code changed
    assert bench.traffic_from_profile("mixed") is None


def test_committed_profiles_carry_a_code_hash_and_traffic():
    profiles = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(profiles) if n.endswith("_traffic.md")]
    assert names
    for n in names:
        text = open(os.path.join(profiles, n)).read()
        assert "decode_code_sha256:" in text and "traffic_bytes_per_launch:" in text, n


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_oracle_layer_times_a_whole_layer(capsys):
    """--oracle-layer: the oracle over every (request, KV head) pair of one
    layer, all threads and one thread, one JSON line; no GPU involved."""
    import json
    bench.oracle_layer("tiny", 0, runs=1)
    line = [x for x in capsys.readouterr().out.splitlines() if x.startswith("{")][-1]
    d = json.loads(line)
    assert d["workload"] == "tiny" and d["runs"] == 1 and d["cores"] >= 1
    assert d["kv_bytes"] == 1281 * 256          # the tiny lengths, 1 KV head, D 64, bf16
    assert d["us_all_cores"] > 0 and d["us_one_thread"] > 0
