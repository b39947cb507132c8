"""Host logic of bench.py that decides whether a committed counter summary
still describes the kernel: the source hash ignores comments and layout
whitespace, and sees every change to the code."""
import os

import bench


def _sha(tmp_path, monkeypatch, text):
    d = tmp_path / "compaction_dp_score_amd" / "csrc"
    d.mkdir(parents=True, exist_ok=True)
    (d / "k.hip").write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNELS, "probe_workload", ("k", ["k.hip"]))
    return bench.kernel_sources_sha("probe_workload")


BASE = 'int f(int a) {  // add one\n  return a + 1; /* x */\n}\nconst char* s = "a // b";\n'


def test_comments_and_whitespace_do_not_change_the_hash(tmp_path, monkeypatch):
    h0 = _sha(tmp_path, monkeypatch, BASE)
    h1 = _sha(tmp_path, monkeypatch, BASE.replace("// add one", "// the successor")
              .replace("/* x */", "/* a longer\n   block comment */").replace("  return", "    return"))
    assert h0 == h1


def test_code_changes_change_the_hash(tmp_path, monkeypatch):
    h0 = _sha(tmp_path, monkeypatch, BASE)
    assert _sha(tmp_path, monkeypatch, BASE.replace("a + 1", "a + 2")) != h0
    assert _sha(tmp_path, monkeypatch, BASE.replace('"a // b"', '"a // c"')) != h0   # in a string
    assert os.path.basename(bench.__file__) == "bench.py"


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus N with N > 1 exits with a message
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.abspath(bench.__file__))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""
