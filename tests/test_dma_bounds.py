"""Every direct-to-LDS buffer load of the bf16 tile kernel stays inside what
it may touch (CPU only): tests/dma_replay.cpp runs the kernel's own address
arithmetic on the host for every tile, wave, lane and load instruction of
launches in each shipped tile shape (see its header).  The same replay built
against copies of the kernel source with a planted address mistake must
report failures, so the checks have teeth."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_ffn_04_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
REPLAY = os.path.join(ROOT, "tests", "dma_replay.cpp")

# (file, text, planted replacement): a lane's chunk one past its row, the
# token extent covering the whole tile height whatever its rows, an LDS
# destination one row too far
MUTATIONS = [
    ("gemm_bf16.hip", "voff[i] = static_cast<int>(off) + c * 16;", "voff[i] = static_cast<int>(off) + c * 16 + 16;"),
    ("gemm_bf16.hip", ": static_cast<int>((b.vrows < cap ? b.vrows : cap) * rowb);", ": static_cast<int>(cap * rowb);"),
    ("gemm_bf16.hip", "dst[i] = row0 * CH * 16;", "dst[i] = (row0 + 1) * CH * 16;"),
]


def _build_and_run(tmp_path, csrc, tag):
    exe = tmp_path / f"replay_{tag}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-Wno-inline-asm", REPLAY, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)


def test_tile_loads_stay_in_bounds(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = _build_and_run(tmp_path, CSRC, "shipped")
    assert out.returncode == 0 and "failures 0" in out.stdout, out.stdout[-3000:]


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_planted_address_mistakes_are_caught(tmp_path, i):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    fname, old, new = MUTATIONS[i]
    mut = tmp_path / "csrc"
    shutil.copytree(CSRC, mut)
    src = (mut / fname).read_text()
    assert src.count(old) == 1, f"mutation site not found: {old}"
    (mut / fname).write_text(src.replace(old, new))
    out = _build_and_run(tmp_path, str(mut), f"mut{i}")
    assert out.returncode != 0 and "failures 0" not in out.stdout, out.stdout[-2000:]
