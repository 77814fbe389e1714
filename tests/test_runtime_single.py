"""One HIP runtime per process: loading libharp.so must reuse the HIP
runtime that torch ships, never map a second copy (two runtimes in one
process crash on the first cross-runtime stream or allocation)."""
import subprocess
import sys
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
sys.path.insert(0, %r)
import rotated_bit_amd
libs = set()
for line in open('/proc/self/maps'):
    parts = line.split()
    if len(parts) >= 6 and ('libamdhip64' in parts[-1] or 'libhsa-runtime64' in parts[-1]):
        libs.add(parts[-1])
print('\n'.join(sorted(libs)))
"""


def test_single_hip_runtime_and_it_is_torchs():
    out = subprocess.run([sys.executable, "-c", PROBE % ROOT], capture_output=True,
                         text=True, check=True).stdout.split()
    hip = [p for p in out if "libamdhip64" in p]
    hsa = [p for p in out if "libhsa-runtime64" in p]
    assert len(hip) == 1 and len(hsa) == 1, out
    import torch
    tdir = os.path.dirname(torch.__file__)
    assert hip[0].startswith(tdir), hip
