"""Host logic of bench.py (no GPU): the refusal of more than one GPU and the
source hash that keys the committed HBM-traffic counters to the code they
were taken on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _hash_of(tmp_path, texts, monkeypatch):
    for rel, text in zip(bench.TRAFFIC_SOURCES, texts):
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text(text, encoding="utf-8")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return bench.kernel_sources_sha256()


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    code = ["int f(int x) {\n  return x + 1;\n}\n", "#define K 4\n"]
    base = _hash_of(tmp_path, code, monkeypatch)
    commented = ["// what f does\nint f(int x) {  // trailing note\n\n  return x + 1;  /* inline */\n}\n",
                 "/* header\n   block */\n#define K 4\n"]
    assert _hash_of(tmp_path, commented, monkeypatch) == base
    changed = ["int f(int x) {\n  return x + 2;\n}\n", "#define K 4\n"]
    assert _hash_of(tmp_path, changed, monkeypatch) != base
    moved = ["#define K 4\n", "int f(int x) {\n  return x + 1;\n}\n"]  # order of the files matters
    assert _hash_of(tmp_path, moved, monkeypatch) != base


def test_traffic_summary_is_read_only_for_matching_code(tmp_path, monkeypatch):
    code = ["int g() { return 0; }\n", "#define D 128\n"]
    h = _hash_of(tmp_path, code, monkeypatch)
    summary = tmp_path / "traffic.md"
    summary.write_text(f"- `kernel_sources_sha256`: `{h}`\n- `fetch_bytes_per_launch`: `100`\n"
                       "- `write_bytes_per_launch`: `23`\n", encoding="utf-8")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.profiled_traffic() == 123
    _hash_of(tmp_path, ["int g() { return 1; }\n", "#define D 128\n"], monkeypatch)
    assert bench.profiled_traffic() is None
