"""CPU: the product path has no fallback.

Without the built library, importing the package fails with a message that
says how to build it; and nothing in the package (binding, build script, HIP
sources) refers to the oracle, so no call can reach a CPU implementation.
"""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "selective_state_space_softplus_amd")


def test_import_fails_without_the_library(tmp_path):
    pkg = tmp_path / "selective_state_space_softplus_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), pkg / "__init__.py")
    code = f"import sys; sys.path.insert(0, {str(tmp_path)!r}); import selective_state_space_softplus_amd"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "is not built" in r.stderr, r.stderr[-2000:]


def test_package_never_refers_to_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for name in files:
            if name.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, name), encoding="utf-8").read()
                assert "oracle" not in text.lower(), os.path.join(dirpath, name)


def test_traffic_record_is_readable_by_the_bench():
    """profiles/traffic.json holds the counter-measured HBM bytes of the scan kernel under the key bench.py looks up,
    with the fields it reports; whether its source hash is current is the bench's business (it reports null
    otherwise)."""
    import json

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    rec = json.load(open(os.path.join(root, "profiles", "traffic.json")))["scan_seq"]
    for key in ("kernel", "bytes_per_launch", "algorithmic_bytes", "source_hash", "fetch_scale", "write_scale"):
        assert key in rec, key
    assert 0.9 < rec["bytes_per_launch"] / rec["algorithmic_bytes"] < 3.0
