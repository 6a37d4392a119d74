"""The product path stands alone (no GPU needed): without the built library the binding raises
instead of computing anything, and neither the package nor the library it loads refers to the
oracle, which is test infrastructure only."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "normalization_reductions_amd")


def test_binding_raises_without_the_library(tmp_path):
    # a fresh interpreter whose NORMRED_LIB names a file that does not exist: the first call
    # must raise, naming the build step, and must not fall back to another implementation
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import torch\n"
        "import normalization_reductions_amd as nra\n"
        "try:\n"
        "    nra.inorm_forward(torch.zeros(1, 1, 8))\n"
        "except RuntimeError as e:\n"
        "    print('RAISED', e)\n"
        "else:\n"
        "    print('NO ERROR')\n" % ROOT)
    env = dict(os.environ, NORMRED_LIB=str(tmp_path / "missing" / "libnormred.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert "RAISED" in r.stdout and "not built" in r.stdout


def test_package_sources_do_not_use_the_oracle():
    pat = re.compile(r"\boracle\b")
    for dirpath, _, files in os.walk(PKG):
        if "_build" in dirpath or "__pycache__" in dirpath:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                # build.py also compiles oracle.c, for the host-sanitizer test only
                # (build_host_asan); nothing it builds into libnormred.so comes from there
                if f == "build.py":
                    continue
                with open(os.path.join(dirpath, f), encoding="utf-8") as fh:
                    assert not pat.search(fh.read()), "%s refers to the oracle" % os.path.join(dirpath, f)


def test_library_does_not_link_the_oracle():
    lib = os.path.join(PKG, "libnormred.so")
    if not os.path.exists(lib):
        import pytest

        pytest.skip("libnormred.so not built")
    out = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    needed = re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out)
    assert needed, out
    assert not any("oracle" in n for n in needed), needed
    syms = subprocess.run(["readelf", "--dyn-syms", "-W", lib], capture_output=True, text=True,
                          check=True).stdout
    assert not re.search(r"\bor_[a-z_]+\b", syms), "the library exports or imports oracle symbols"
