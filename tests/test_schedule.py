"""Host build of the tile scheduler header (the same file the kernels use):
bijection of the XCD slot map, every tile visited exactly once for many grid
shapes, and XCD locality of the 4096^3 launch."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_schedule_bijection_and_locality(tmp_path):
    exe = tmp_path / "schedule_check"
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "bf16_gemm_fp32_amd", "csrc"),
                    os.path.join(ROOT, "tests", "schedule_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout[-2000:]
    lines = out.stdout.strip().splitlines()
    assert lines[-1] == "OK"
    # each XCD's 32 tiles of the 16x16 grid form a 4 x 8 block
    xcd = [l for l in lines if l.startswith("xcd")]
    assert len(xcd) == 8
    for l in xcd:
        _, _, _, rows, _, cols = l.split()
        assert (int(rows), int(cols)) == (4, 8), l
