"""Host-side checks of scheduling logic shared with the device code (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_dispatch_amd", "csrc")
HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_tile_schedules_cover_every_tile_once(tmp_path):
    exe = tmp_path / "tile_split"
    src = os.path.join(ROOT, "tests", "host", "tile_split.cpp")
    subprocess.run([HIPCC, "--cuda-host-only", "-O1", "-I", CSRC, "-o", str(exe), src], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
