"""Every direct-to-LDS load and every LDS read of the MXFP4 LDS-staged kernel
stays inside what it may touch and reads what the arithmetic needs (CPU
only): tests/mx_lds_replay.cpp runs the kernel's own address arithmetic on
the host for every workgroup, wave, lane, load and stage of launches in
several shapes (see its header).  The same replay built against copies of
the kernel source with a planted address mistake must report failures, so
the checks have teeth."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_ffn_04_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
REPLAY = os.path.join(ROOT, "tests", "mx_lds_replay.cpp")

# (text, planted replacement) in decode_mx.hip: a code read without the
# bank swizzle, the up rows' scales one row off, a token read swizzled by
# the wrong row, one token load too few for a chunk's rows
MUTATIONS = [
    ("return rl * 128 + (((4 * u + q) ^ ((rl >> 1) & 7)) * 16);", "return rl * 128 + ((4 * u + q) * 16);"),
    ("(N + n0) * KB + b - 32 * KB : n0 * KB + b;", "(N + n0 + 1) * KB + b - 32 * KB : n0 * KB + b;"),
    ("return i * 512 + (((16 * u + 4 * q + m) ^ i) * 16);", "return i * 512 + (((16 * u + 4 * q + m) ^ (i + 1)) * 16);"),
    ("const int n = (left - 4 * wave + 1) / 2;", "const int n = (left - 4 * wave) / 2;"),
]


def _build_and_run(tmp_path, csrc, tag):
    exe = tmp_path / f"mx_replay_{tag}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-Wno-inline-asm", REPLAY, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)


def test_mx_lds_loads_and_reads(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = _build_and_run(tmp_path, CSRC, "shipped")
    assert out.returncode == 0 and "failures 0" in out.stdout.splitlines()[-1], out.stdout[-3000:]


@pytest.mark.parametrize("i", range(len(MUTATIONS)))
def test_planted_mx_address_mistakes_are_caught(tmp_path, i):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    old, new = MUTATIONS[i]
    mut = tmp_path / "csrc"
    shutil.copytree(CSRC, mut)
    src = (mut / "decode_mx.hip").read_text()
    assert src.count(old) == 1, f"mutation site not found: {old}"
    (mut / "decode_mx.hip").write_text(src.replace(old, new))
    out = _build_and_run(tmp_path, str(mut), f"mut{i}")
    assert out.returncode != 0 and "failures 0" not in out.stdout.splitlines()[-1], out.stdout[-2000:]
