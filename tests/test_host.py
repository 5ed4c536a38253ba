"""CPU: the host-side contracts around the library. The product path loads
only the built library (never the oracle, never a CPU fallback) and fails
loudly without it; the benchmark measures one GPU and refuses more."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _py(code, *args, timeout=240):
    return subprocess.run([sys.executable, "-c", code, *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_missing_library_fails_loudly():
    r = _py("import top_index_sparse_amd as sa\n"
            "sa.LIB_PATH = '/nonexistent/libsparse_attn.so'; sa._LIB = None\n"
            "try:\n"
            "    sa.sparse_attn_union_workspace_bytes(8, 64, 2)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "missing" in r.stdout


def test_package_does_not_load_the_oracle():
    r = _py("import sys, top_index_sparse_amd as sa\n"
            "sa.lib()\n"
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))\n")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"
    pkg = os.path.join(ROOT, "top_index_sparse_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
