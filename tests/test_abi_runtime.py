"""The binding loads torch's HIP runtime before libtreeattn, so the process
holds exactly one HIP runtime (checked on the CPU through /proc/self/maps)."""
import os
import subprocess
import sys

from helpers import ROOT


def test_single_hip_runtime_in_process():
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import tree_masked_verify_attn_amd as ta\n"
        "ta.load_library()\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "libs = sorted({ln.split()[-1] for ln in maps if 'libamdhip64' in ln})\n"
        "print(len(libs)); print(libs)\n" % ROOT)
    from tree_masked_verify_attn_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    n = int(out.stdout.splitlines()[0])
    assert n == 1, out.stdout
