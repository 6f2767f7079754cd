"""bench.py on the CPU: more than one GPU is refused with a message and a
non-zero status, before anything touches a GPU; the kernel-source hash that
keys the stored counter data ignores comments only."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_only():
    """The stored counter data stays valid across comment edits and goes
    stale on any code edit."""
    sys.path.insert(0, ROOT)
    import bench
    base = 'int f(int x) { // twice\n  return 2 * x; /* doubled */ }\nconst char* s = "a//b";\n'
    same = '// header\nint f(int x) {\n  return 2 * x; }\n\nconst char* s = "a//b";  // kept\n'
    code = base.replace("2 * x", "3 * x")
    lit = base.replace('"a//b"', '"a// b"')
    assert bench.code_only(base) == bench.code_only(same)
    assert bench.code_only(base) != bench.code_only(code)
    assert bench.code_only(base) != bench.code_only(lit)
