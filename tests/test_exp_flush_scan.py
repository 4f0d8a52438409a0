"""The attention softmax evaluates its exp without flushes when x = 0 or
|x| >= 2^-100.  That equals the flushed definition only if no step of the
reduction and polynomial is subnormal for any such binary32 x in
[-104, 0]; tests/csrc/exp_flush_scan.c checks every one of them on the CPU.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_unflushed_exp_has_no_subnormal_step(tmp_path):
    exe = tmp_path / "scan"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    os.path.join(HERE, "csrc", "exp_flush_scan.c"), "-o", str(exe), "-lm"],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, check=True)
    bad, rmin = r.stdout.split()
    assert int(bad) == 0
    assert float.fromhex(rmin) >= 2.0 ** -100
