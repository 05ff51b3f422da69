"""The C ABI on the CPU: the library loads without a GPU, exports exactly
what include/libmoe.h declares, and its host-side validation returns the
documented status codes before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_ffn_04_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return binding.load()


def test_header_declares_the_path():
    names = declared()
    for n in ["moe_route", "moe_topk", "moe_permute", "moe_permute_workspace_size",
              "moe_grouped_gemm_gateup_swiglu", "moe_grouped_gemm_down", "moe_unpermute_combine",
              "moe_decode_gateup_swiglu", "moe_decode_down", "moe_decode_gateup_swiglu_gather",
              "moe_grouped_gemm_gateup_swiglu_gather", "moe_localize_ids",
              "moe_abi_version", "moe_status_string"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from mixture_experts_ffn_04_amd import binding
    for n in declared():
        assert hasattr(lib, n), n
    assert set(binding.EXPORTS) == set(declared())


def test_version_and_strings(lib):
    assert lib.moe_abi_version() == 1
    for s in range(6):
        assert lib.moe_status_string(s)
    assert b"unknown" in lib.moe_status_string(99)


def test_validation_without_gpu(lib):
    from mixture_experts_ffn_04_amd import binding as B
    P = 4096   # a fake, 16-byte aligned "device" address: validation fails before any use
    # k out of range, E too large, unknown score
    assert lib.moe_topk(P, 10, 8, 0, 0, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_topk(P, 10, 8, 9, 0, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_topk(P, 10, 300, 2, 0, P, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_topk(P, 10, 8, 17, 0, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_topk(P, 10, 8, 2, 7, P, P, None) == B.MOE_ERR_INVALID_ARG
    # d not a multiple of 64, misaligned pointer, null
    assert lib.moe_route(P, P, None, 10, 100, 8, 2, 1, 0, P, P, P, None) == B.MOE_ERR_ALIGNMENT
    assert lib.moe_route(P + 2, P, None, 10, 128, 8, 2, 1, 0, P, P, P, None) == B.MOE_ERR_ALIGNMENT
    assert lib.moe_route(None, P, None, 10, 128, 8, 2, 1, 0, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_route(P, P, None, 10, 128, 8, 2, 5, 0, P, P, P, None) == B.MOE_ERR_INVALID_ARG
    # T = 0 is a valid no-op
    assert lib.moe_route(None, None, None, 0, 128, 8, 2, 1, 0, None, None, None, None) == B.MOE_OK
    assert lib.moe_topk(None, 0, 8, 2, 0, None, None, None) == B.MOE_OK
    # permute workspace
    need = lib.moe_permute_workspace_size(1000, 4, 32)
    assert need >= 4 * 32
    assert lib.moe_permute(P, P, 1000, 128, 32, 4, 1, P, P, P, P, P, P, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_permute(P, P, 1000, 128, 32, 4, 1, P, P, P, P, P, None, need, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_permute(P, P, 1000, 100, 32, 4, 1, P, P, P, P, P, P, need, None) == B.MOE_ERR_ALIGNMENT
    # projections
    for fn in (lib.moe_grouped_gemm_gateup_swiglu, lib.moe_grouped_gemm_down,
               lib.moe_decode_gateup_swiglu, lib.moe_decode_down):
        assert fn(P, P, P, 100, 128, 96, 8, 1, P, None) == B.MOE_ERR_ALIGNMENT
        assert fn(P, P, P, 100, 128, 128, 0, 1, P, None) == B.MOE_ERR_INVALID_ARG
        assert fn(P, P, P, 100, 128, 128, 257, 1, P, None) == B.MOE_ERR_UNSUPPORTED
        assert fn(P, P, None, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG
        assert fn(None, None, None, 0, 128, 128, 8, 1, None, None) == B.MOE_OK
    assert lib.moe_decode_down(P, P, P, 1025, 128, 128, 8, 1, P, None) == B.MOE_ERR_UNSUPPORTED
    for g in (lib.moe_decode_gateup_swiglu_gather, lib.moe_grouped_gemm_gateup_swiglu_gather):
        assert g(P, P, 3, P, P, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG     # rows % k != 0
        assert g(P, None, 2, P, P, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG  # no perm
        assert g(P, P, 2, P, P, 100, 128, 128, 8, 0, P, None) == B.MOE_ERR_UNSUPPORTED     # fp32
        assert g(None, None, 2, None, None, 0, 128, 128, 8, 1, None, None) == B.MOE_OK
    assert lib.moe_localize_ids(P, 10, 0, 0, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids(P, 10, -1, 4, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids(P, 10, 0, 257, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_localize_ids(None, 0, 0, 4, None, None) == B.MOE_OK
    assert lib.moe_localize_ids(None, 10, 0, 4, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids_strided(P, 10, 0, 0, 4, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids_strided(P, 10, 1, 8, 0, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids_strided(P, 10, 0, 2, 257, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_localize_ids_strided(None, 0, 3, 8, 32, None, None) == B.MOE_OK
    assert lib.moe_localize_ids_mapped(P, 10, P, 0, 4, P, None) == B.MOE_ERR_INVALID_ARG      # no experts
    assert lib.moe_localize_ids_mapped(P, 10, P, 64, 0, P, None) == B.MOE_ERR_INVALID_ARG     # none held
    assert lib.moe_localize_ids_mapped(P, -1, P, 64, 8, P, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_localize_ids_mapped(P, 10, P, 257, 8, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_localize_ids_mapped(P, 10, P, 64, 257, P, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_localize_ids_mapped(P, 10, None, 64, 8, P, None) == B.MOE_ERR_INVALID_ARG  # no map
    assert lib.moe_localize_ids_mapped(None, 0, None, 64, 8, None, None) == B.MOE_OK
    g = lib.moe_decode_gateup_swiglu_gather
    assert g(P, P, 3, P, P, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG     # rows % k != 0
    assert g(P, P, 0, P, P, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG     # k < 1
    assert g(P, None, 2, P, P, 100, 128, 128, 8, 1, P, None) == B.MOE_ERR_INVALID_ARG  # no perm
    assert g(P, P, 2, P, P, 100, 128, 128, 8, 0, P, None) == B.MOE_ERR_UNSUPPORTED     # fp32
    assert g(P, P, 2, P, P, 1026, 128, 128, 8, 1, P, None) == B.MOE_ERR_UNSUPPORTED    # rows > 1024
    assert g(P, P, 2, P, P, 100, 128, 96, 8, 1, P, None) == B.MOE_ERR_ALIGNMENT
    assert g(None, None, 2, None, None, 0, 128, 128, 8, 1, None, None) == B.MOE_OK
    assert lib.moe_unpermute_combine(P, P, P, None, 10, 100, 2, 1, P, None) == B.MOE_ERR_ALIGNMENT
    assert lib.moe_unpermute_combine(P, P, P, None, 10, 128, 0, 1, P, None) == B.MOE_ERR_INVALID_ARG


C_CLIENT = r"""
#include <stdio.h>
#include <string.h>
#include "libmoe.h"
int main(void) {
  int fake = 0;
  void* p = (void*)((((unsigned long)&fake) + 4096) & ~15ul);   /* aligned, never dereferenced */
  if (moe_abi_version() != 1) return 1;
  if (strcmp(moe_status_string(MOE_ERR_ALIGNMENT), "misaligned pointer or size not a multiple of 64") != 0) return 2;
  /* host-side validation answers before any launch */
  if (moe_route(p, p, NULL, 10, 100, 8, 2, MOE_BF16, MOE_SCORE_SOFTMAX, (float*)p, (int32_t*)p, (float*)p, NULL)
      != MOE_ERR_ALIGNMENT) return 3;
  if (moe_topk((const float*)p, 10, 8, 9, MOE_SCORE_SOFTMAX, (int32_t*)p, (float*)p, NULL) != MOE_ERR_INVALID_ARG)
    return 4;
  if (moe_permute_workspace_size(1000, 4, 32) < 4 * 32) return 5;
  printf("ok\n");
  return 0;
}
"""


def test_header_is_plain_c_and_links(tmp_path):
    """include/libmoe.h compiles as strict C99 and C++11, and a C program
    links against libmoe.so and gets the documented answers (no GPU use)."""
    import shutil
    import subprocess
    from mixture_experts_ffn_04_amd import binding
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "client.c"
    src.write_text(C_CLIENT)
    inc = os.path.join(ROOT, "include")
    for cmd in (["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", inc, "-fsyntax-only", str(src)],
                ["g++", "-std=c++11", "-Wall", "-Wextra", "-Werror", "-I", inc, "-fsyntax-only", "-x", "c++",
                 str(src)]):
        subprocess.run(cmd, check=True)
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libmoe.so not built")
    exe = tmp_path / "client"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-L", libdir, "-l:libmoe.so",
                    "-Wl,-rpath," + libdir, "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout, out.stderr)
