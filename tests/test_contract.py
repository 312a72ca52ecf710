"""Host-side contract checks: no silent fallback without the HIP library, and
bench.py refuses more than one GPU with a message (no GPU needed)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_package_without_library_fails_loudly(tmp_path):
    """A copy of the package without libmla_decode.so raises on import; nothing falls back to the CPU."""
    pkg = tmp_path / "mla_decode_02_amd"
    shutil.copytree(os.path.join(ROOT, "mla_decode_02_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import mla_decode_02_amd"], cwd=tmp_path, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libmla_decode.so" in r.stderr and "no non-HIP fallback" in r.stderr


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
