"""moe_permute_noalloc (the sort with the library's own per-GPU scratch, for
callers that cannot allocate) against moe_permute with a caller workspace:
bit-identical outputs on two calls in a row, the second with a smaller
input, both through the C ABI."""
import numpy as np
import pytest
import torch

import moe_workloads as W

pytestmark = pytest.mark.gpu


def _run(B, fn, ids, x, E, gpu):
    T, k = ids.shape
    P = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device=gpu)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=gpu)
    perm = torch.full((P,), -7, dtype=torch.int32, device=gpu)
    inv = torch.full((P,), -7, dtype=torch.int32, device=gpu)
    xp = torch.zeros(P, x.shape[1], dtype=x.dtype, device=gpu)
    ids_d = torch.from_numpy(ids).to(gpu)
    if fn == "ws":
        ws = torch.empty(max(1, B.permute_workspace_size(T, k, E)), dtype=torch.uint8, device=gpu)
        B.permute(ids_d, x, E, counts, offsets, perm, inv, xp, ws)
    else:
        B.permute_noalloc(ids_d, x, E, counts, offsets, perm, inv, xp)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (counts, offsets, perm, inv)] + [xp.view(torch.int16).cpu().numpy()]


@pytest.mark.parametrize("T,E,k,s", [(16384, 256, 8, 1.0), (8192, 128, 8, 1.1), (4096, 8, 2, None)])
def test_permute_noalloc_matches_workspace_form(gpu, T, E, k, s):
    from mixture_experts_ffn_04_amd import binding as B
    # the larger input first, then a smaller one: the second call reuses the
    # scratch the first left behind
    for TT in (T, T // 3 + 5):
        ids = W.gen_ids(TT, E, k, seed=TT + E, zipf_s=s)
        x = torch.from_numpy(W.gen_matrix((TT, 64), seed=TT).view(np.int16)).to(gpu).view(torch.bfloat16)
        ref = _run(B, "ws", ids, x, E, gpu)
        got = _run(B, "noalloc", ids, x, E, gpu)
        for name, a, b in zip(("counts", "offsets", "perm", "inv_perm", "x_perm"), ref, got):
            assert (a == b).all(), f"T={TT} E={E}: {name} differs"


def test_permute_noalloc_rejects_sizes_past_its_scratch(gpu):
    from mixture_experts_ffn_04_amd import binding as B
    lib = B.load()
    P = 4096
    # 256 experts: at most 1024 chunks of 1024 pairs fit the 1 MiB scratch
    T, k = 1024 * 1024 // 8 + 1, 8
    st = lib.moe_permute_noalloc(P, None, T, 0, 256, k, B.MOE_BF16, P, P, P, P, None, None)
    assert st == B.MOE_ERR_WORKSPACE


def test_permute_noalloc_in_a_graph(gpu):
    """The call its callers need: captured in a HIP graph (no allocation, no
    memset inside) and replayed several times with new ids and other work on
    the stream in between; every replay equals the workspace form."""
    from mixture_experts_ffn_04_amd import binding as B
    T, E, k = 3000, 64, 4
    x = torch.from_numpy(W.gen_matrix((T, 64), seed=5).view(np.int16)).to(gpu).view(torch.bfloat16)
    ids_d = torch.from_numpy(W.gen_ids(T, E, k, seed=1)).to(gpu)
    P = T * k
    outs = [torch.empty(E, dtype=torch.int32, device=gpu), torch.empty(E + 1, dtype=torch.int32, device=gpu),
            torch.empty(P, dtype=torch.int32, device=gpu), torch.empty(P, dtype=torch.int32, device=gpu)]
    xp = torch.empty(P, 64, dtype=torch.bfloat16, device=gpu)
    side = torch.cuda.Stream(device=gpu)
    side.wait_stream(torch.cuda.current_stream(gpu))
    with torch.cuda.stream(side):
        B.permute_noalloc(ids_d, x, E, *outs, xp)          # the device's scratch address is looked up here
    torch.cuda.current_stream(gpu).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        B.permute_noalloc(ids_d, x, E, *outs, xp)
    for rep in range(4):
        ids = W.gen_ids(T, E, k, seed=10 + rep, zipf_s=1.2 if rep % 2 else None)
        ids_d.copy_(torch.from_numpy(ids))
        g.replay()
        torch.cuda.synchronize()
        got = [t.cpu().numpy() for t in outs] + [xp.view(torch.int16).cpu().numpy()]
        ref = _run(B, "ws", ids, x, E, gpu)
        for name, a, b in zip(("counts", "offsets", "perm", "inv_perm", "x_perm"), ref, got):
            assert (a == b).all(), f"replay {rep}: {name} differs"
        torch.sum(x.float())                                  # other work between replays
