"""The product path stands alone: nothing in the package or the C sources
reads the oracle, and without the built library the binding raises instead of
computing anything on the CPU."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "kv_cache_compression_quantize_amd")


def test_package_and_kernels_never_reference_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b)|oracle/|#include[^\n]*oracle", re.M)
    for base, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(base, f), encoding="utf-8").read()
                assert not pat.search(text), os.path.join(base, f)
    assert not pat.search(open(os.path.join(ROOT, "include", "aqkv.h"), encoding="utf-8").read())


def test_missing_library_raises():
    code = ("from kv_cache_compression_quantize_amd import aqkv\n"
            "try:\n"
            "    aqkv.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    env = dict(os.environ, AQKV_LIB=os.path.join(ROOT, "no_such_dir", "libaqkv.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("raised:"), r.stdout
