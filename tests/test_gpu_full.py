"""GPU parity at the full workload sizes (Mixtral-, gpt-oss- and
DeepSeek-shaped layers and the fine-grained Zipf layer), through the C ABI.

What is compared:
  * router logits for every token against the float64 oracle, within the
    fp32 dot-product error bound;
  * routing for every token (bit-exact away from near-ties, valid top-k at
    near-ties);
  * the sort by expert, bit-exact against the oracle, on the oracle's own
    routing of the same inputs;
  * properties of every GPU output that hold at any size (counts, offsets,
    bijective stable permutation, weights summing to 1);
  * sampled rows / tokens of H, Y_perm and y against the oracle evaluated
    one row or token at a time.
"""
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import moe_workloads as W
from oracle import moe_oracle as O
from tests import gpu_util as U

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["c2", "c3_t1", "c3_t8", "c3_t32", "c3_t64", "c4", "c5"]
SAMPLE_TOKENS = {"c2": 24, "c4": 64, "c5": 16}
SAMPLE_ROWS = {"c2": 24, "c4": 64, "c5": 24}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _upload(wl):
    """Generate the workload (experts in a thread pool) straight to the GPU."""
    from mixture_experts_ffn_04_amd import MoeLayer, MoeWeights
    dt = wl.dtype
    x = W.gen_x(wl)
    wr, bias = W.gen_router(wl)
    tdt = U.torch_dtype(dt)
    gu = torch.empty(wl.E, 2 * wl.f, wl.d, dtype=tdt, device="cuda")
    dn = torch.empty(wl.E, wl.d, wl.f, dtype=tdt, device="cuda")
    for e, g, w in W.iter_experts(wl):
        gu[e].copy_(U.dev_tensor(g, dt))
        dn[e].copy_(U.dev_tensor(w, dt))
    sh = W.gen_shared(wl)
    weights = MoeWeights(U.dev_tensor(wr, dt), None if bias is None else torch.from_numpy(bias).cuda(), gu, dn,
                         None if sh is None else U.dev_tensor(sh[0], dt),
                         None if sh is None else U.dev_tensor(sh[1], dt))
    return x, wr, bias, sh, weights


def _fetch_many(wl, experts):
    """Oracle-side expert weights regenerated from the seeds, kept in their
    2-byte storage format (decoded to float64 one expert at a time by
    _f64_expert, so the DeepSeek-shaped layer fits in host memory)."""
    with ThreadPoolExecutor(W.default_threads()) as ex:
        return dict(zip(experts, ex.map(lambda e: W.gen_expert(wl, e), experts)))


def _f64_expert(wl, stored, e):
    g, w = stored[e]
    return W.values(g, wl.dtype), W.values(w, wl.dtype)


@pytest.mark.parametrize("name", FULL)
def test_full_size(gpu, name):
    from mixture_experts_ffn_04_amd import MoeLayer, binding as B
    wl = W.get(name)
    t0 = time.time()
    log(f"[{name}] generating and uploading")
    x, wr, bias, sh, weights = _upload(wl)
    x_dev = U.dev_tensor(x, wl.dtype)
    x64 = W.values(x, wl.dtype)
    wr64 = W.values(wr, wl.dtype)
    log(f"[{name}] oracle routing ({time.time() - t0:.1f}s)")
    L = O.router_logits(x64, wr64, bias)
    ids_ref, w_ref = O.route(L, wl.k, wl.score)
    E, k, T, P = wl.E, wl.k, wl.T, wl.P

    # ---- the layer on the GPU (decode calls for the small-batch workload)
    log(f"[{name}] GPU layer")
    layer = B.MoeLayer(weights, k, wl.score)
    y = layer.forward(x_dev)
    torch.cuda.synchronize()
    g_logits = layer.logits.cpu().numpy().astype(np.float64)
    g_ids = layer.ids.cpu().numpy()
    g_w = layer.wts.cpu().numpy().astype(np.float64)
    g_counts = layer.counts.cpu().numpy()
    g_off = layer.offsets.cpu().numpy()
    g_perm = layer.perm.cpu().numpy().astype(np.int64)
    g_inv = layer.inv_perm.cpu().numpy().astype(np.int64)
    g_y = U.host_values(y)

    # logits and routing, every token
    bound = O.logit_error_bound(x64, wr64, bias)
    assert (np.abs(g_logits - L) <= bound).all(), "router logits outside the fp32 error bound"
    same = U.routing_agreement(g_ids, L, x64, wr64, bias, k)
    log(f"[{name}] routing: {int((~same).sum())} near-tie tokens differ of {T}")
    assert np.abs(g_w[same] - w_ref[same]).max() <= U.WEIGHT_ABS
    assert np.abs(g_w.sum(1) - 1).max() <= 1e-6

    # properties of the GPU sort at full size
    flat = g_ids.reshape(-1).astype(np.int64)
    assert (g_counts == np.bincount(flat, minlength=E)).all()
    assert g_off[0] == 0 and (np.diff(g_off) == g_counts).all() and g_off[-1] == P
    assert (np.sort(g_perm) == np.arange(P)).all() and (g_inv[g_perm] == np.arange(P)).all()
    grp = flat[g_perm]
    assert (np.diff(grp) >= 0).all()
    same_grp = np.diff(grp) == 0
    assert (np.diff(g_perm)[same_grp] > 0).all(), "sort is not stable"

    # ---- the sort on the oracle's routing: bit-exact
    log(f"[{name}] permute on oracle routing")
    rc, ro, rp, ri = O.permute(ids_ref, E)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(P, dtype=torch.int32, device="cuda")
    inv = torch.empty(P, dtype=torch.int32, device="cuda")
    xp = torch.empty(P, wl.d, dtype=x_dev.dtype, device="cuda")
    ws = torch.empty(B.permute_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    B.permute(_i32(ids_ref), x_dev, E, counts, offsets, perm, inv, xp, ws)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == rc).all() and (offsets.cpu().numpy() == ro).all()
    assert (perm.cpu().numpy() == rp).all() and (inv.cpu().numpy() == ri).all()
    rng = np.random.default_rng(7)
    chk = rng.choice(P, size=min(P, 512), replace=False)
    assert (U.host_bits(xp[torch.from_numpy(chk).cuda()]) == np.asarray(x)[rp[chk] // k]).all()

    # ---- the projections on that (oracle-routed) grouping, sampled rows
    decode = layer.use_decode(T)
    h = torch.empty(P, wl.f, dtype=x_dev.dtype, device="cuda")
    yp = torch.empty(P, wl.d, dtype=x_dev.dtype, device="cuda")
    B.gateup_swiglu(xp, weights.w_gate_up, offsets, h, decode)
    B.down(h, weights.w_down, offsets, yp, decode)
    torch.cuda.synchronize()
    nrows = SAMPLE_ROWS.get(name, P)
    rows = np.sort(rng.choice(P, size=min(P, nrows), replace=False))
    row_e = np.searchsorted(ro, rows, side="right") - 1
    wts = _fetch_many(wl, sorted(set(row_e.tolist())))
    log(f"[{name}] sampled rows: {rows.size} over {len(wts)} experts ({time.time() - t0:.1f}s)")
    h_rows = U.host_values(h[torch.from_numpy(rows).cuda()])
    h_ref = np.empty_like(h_rows)
    y_ref = np.empty((rows.size, wl.d))
    for e in sorted(set(row_e.tolist())):
        gu64, dn64 = _f64_expert(wl, wts, e)
        for i in np.nonzero(row_e == e)[0]:
            h_ref[i] = O.gate_up_swiglu(x64[rp[rows[i]] // k][None], gu64)[0]
            y_ref[i] = O.down(h_ref[i][None], dn64)[0]          # the oracle's own H
        del gu64, dn64
    U.assert_close(h_rows, h_ref, wl.dtype, f"{name} H rows")
    U.assert_close(U.host_values(yp[torch.from_numpy(rows).cuda()]), y_ref, wl.dtype, f"{name} Y_perm rows")

    # ---- whole layer, sampled tokens with identical routing
    ntok = SAMPLE_TOKENS.get(name, T)
    cand = np.nonzero(same)[0]
    toks = np.sort(rng.choice(cand, size=min(cand.size, ntok), replace=False))
    need = sorted(set(ids_ref[toks].reshape(-1).tolist()))
    wts = _fetch_many(wl, need)
    shared = None if sh is None else (W.values(sh[0], wl.dtype), W.values(sh[1], wl.dtype))
    y_ref = O.moe_layer_eager(x64[toks], ids_ref[toks], w_ref[toks], lambda e: _f64_expert(wl, wts, e), E, shared)
    log(f"[{name}] sampled tokens: {toks.size} ({time.time() - t0:.1f}s)")
    U.assert_close(g_y[toks], y_ref, wl.dtype, f"{name} layer")

    # ---- decode workloads: the decode and grouped calls agree
    if decode:
        grouped = B.MoeLayer(weights, k, wl.score, mode="grouped")
        yg = U.host_values(grouped.forward(x_dev))
        torch.cuda.synchronize()
        U.assert_close(g_y, yg, wl.dtype, f"{name} decode vs grouped")
    log(f"[{name}] done ({time.time() - t0:.1f}s)")
    del weights, layer, xp, h, yp
    torch.cuda.empty_cache()
