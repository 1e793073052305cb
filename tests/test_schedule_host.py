"""Host logic of the persistent scheduler, checked on the CPU: the down-tile
claim map (which tiles are cut into K halves and where their halves sit in
the per-XCD claim ranges) is compiled from the library's header with hipcc
as a host program and run exhaustively over tile counts and grid sizes."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_down_claim_map_is_a_bijection(tmp_path):
    exe = tmp_path / "claim_map_check"
    src = os.path.join(HERE, "host", "claim_map_check.cpp")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "0 violations" in out.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_expert_aligned_tile_order_is_a_bijection(tmp_path):
    exe = tmp_path / "expert_tile_check"
    src = os.path.join(HERE, "host", "expert_tile_check.cpp")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", src, "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert " 0 violations" in out.stdout
