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


def _gemv_ring_stream(QC, NB, D, ntile):
    """Model of the weight ring of the workgroup weight-streaming GEMV (fp8_gemv_run): the
    blocks each load fetches and each MFMA step reads, for ntile tiles of QC column quads x
    NB blocks.  A ring no deeper than a quad's slice walks quad by quad in steps of D; a ring
    of D = 2 NB walks passes of D / NB quads.  Returns the blocks read, in order, as (tile,
    block); raises on a load outside the tile stream or a step that reads the wrong block."""
    NBT = QC * NB
    slots = [None] * D

    def fetch(n, tl):
        # stream position tl of tile n: this tile's block, else the next tile's (after the
        # last tile: blocks of the same tile that are read again and go unused)
        if tl < NBT:
            return (n, tl)
        tt = tl - NBT
        assert tt < D - 1 and tt < NBT, (QC, NB, D, tl)
        if n + 1 < ntile:
            return (n + 1, tt)
        # quad tt // NB, block tt % NB from the re-read base
        base = 0 if D > NB else (QC - 1) * NB + NB - D  # the tile's start / last quad's block NB - D
        again = base + (tt // NB) * NB + tt % NB
        assert 0 <= again < NBT, (QC, NB, D, again)
        return ("again", again)

    for j in range(D - 1):
        slots[j] = fetch(0, j)
    read = []
    for n in range(ntile):
        if D <= NB:
            steps = [(c * NB + i0 + j, j) for c in range(QC) for i0 in range(0, NB, D) for j in range(D)]
        else:
            steps = [(p * D + j, j) for p in range(QC // (D // NB)) for j in range(D)]
        for t, j in steps:
            slots[(j + D - 1) % D] = fetch(n, t + D - 1)
            assert slots[j] == (n, t), (QC, NB, D, n, t, slots[j])
            read.append((n, t))
    return read


@pytest.mark.parametrize("QC,NB,D", [(1, 4, 4), (2, 4, 4), (4, 4, 4), (1, 8, 4), (2, 8, 4), (4, 8, 4), (1, 8, 8),
                                     (2, 8, 8), (4, 8, 8), (2, 4, 8), (4, 4, 8)])
def test_gemv_weight_ring_reads_every_block_once_in_bounds(QC, NB, D):
    for ntile in (1, 2, 3, 5):
        read = _gemv_ring_stream(QC, NB, D, ntile)
        assert read == [(n, t) for n in range(ntile) for t in range(QC * NB)]
