"""The product path stands on the HIP library alone: it never reaches the oracle, and it
fails loudly, with no fallback, when the library is not there."""
import os
import re
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
PACKAGE = ROOT / "attention_guided_eviction_amd"


def test_package_sources_never_reach_the_oracle():
    offenders = []
    for path in sorted(PACKAGE.rglob("*")):
        if path.suffix not in {".py", ".hip", ".h", ".cpp"} or "_build" in path.parts:
            continue
        text = path.read_text()
        if re.search(r"^\s*(from|import)\s+oracle\b", text, flags=re.M) or re.search(r'#include\s+"[^"]*oracle', text):
            offenders.append(str(path.relative_to(ROOT)))
    assert not offenders, offenders


def test_missing_library_raises_instead_of_falling_back(tmp_path):
    code = (
        "from attention_guided_eviction_amd import bkv\n"
        "try:\n"
        "    bkv.load()\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('loaded')\n"
    )
    env = dict(os.environ, BKV_LIBRARY=str(tmp_path / "absent" / "libbkv.so"))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("raised:") and "is not built" in out.stdout, out.stdout
