"""Helpers shared by the GPU tests: moving storage-format arrays to and from
the device, tolerances, near-tie aware routing comparison and whole-layer
parity on every token."""
from __future__ import annotations

import functools

import numpy as np
import torch

import moe_workloads as W
from oracle import moe_oracle as O

# Tolerances for the layer outputs against the float64 oracle.
BF16_MAX_REL = 2e-2        # max|err| <= 2e-2 * max|ref|
BF16_MEAN_REL = 5e-3       # sum|err| / sum|ref| <= 5e-3
F32_MAX_REL = 1e-4         # max|err| <= 1e-4 * max|ref|
WEIGHT_ABS = 1e-5          # routing weights (fp32 logits -> fp32 weights)


def dev_tensor(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array (bf16 bits as uint16, or fp32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host_values(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 values."""
    if t.dtype == torch.bfloat16:
        return W.values(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    return t.detach().cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def assert_close(got, ref, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    if scale == 0:
        assert err.max() == 0, f"{what}: expected zeros"
        return
    if dtype == "bf16":
        assert err.max() <= BF16_MAX_REL * scale, f"{what}: max err {err.max():.3e} > {BF16_MAX_REL}*{scale:.3e}"
        mean_rel = err.sum() / np.abs(ref).sum()
        assert mean_rel <= BF16_MEAN_REL, f"{what}: mean rel err {mean_rel:.3e}"
    else:
        assert err.max() <= F32_MAX_REL * scale, f"{what}: max err {err.max():.3e} > {F32_MAX_REL}*{scale:.3e}"


def routing_agreement(gpu_ids, ref_logits, x, w_router, bias, k, max_frac=1e-3):
    """Compare GPU routing with the oracle's (float64 logits, selection in
    fp32).  The GPU accumulates the fp32 logits in another order, so where
    two candidates are closer than the fp32 dot-product error bound either
    choice is correct.  Tokens whose selection margin exceeds twice the
    bound must match bit-exactly (ids and order); any other token may
    differ only if the GPU's choice is a valid top-k (set and order) for
    some logits within the bound of the exact ones.  Returns the mask of
    tokens whose ids match exactly."""
    gpu_ids = np.asarray(gpu_ids)
    ref_ids, _ = O.route(ref_logits, k, "softmax")
    b = O.logit_error_bound(x, w_router, bias)                  # [T, E]
    margin = O.topk_margin(ref_logits, k)
    same = (gpu_ids == ref_ids).all(axis=1)
    E = ref_logits.shape[1]
    for t in np.nonzero(~same)[0]:
        assert margin[t] <= 2 * b[t].max(), f"token {t}: routing differs away from a near-tie"
        sel = gpu_ids[t].astype(np.int64)
        assert len(set(sel.tolist())) == k and sel.min() >= 0 and sel.max() < E
        L, bt = ref_logits[t], b[t]
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            assert (L[sel] + bt[sel]).min() >= (L[rest] - bt[rest]).max(), f"token {t}: not a top-{k} set"
        for j in range(k - 1):
            assert L[sel[j]] + bt[sel[j]] >= L[sel[j + 1]] - bt[sel[j + 1]], f"token {t}: order"
    assert (~same).mean() <= max_frac, f"{(~same).sum()} of {same.size} tokens route differently"
    return same


def check_layer(layer, wl, x, wr, bias, expert_weights, shared, y, what: str, tokens=None):
    """Whole-layer parity with no token left out.

    1. The GPU's fp32 logits lie within the fp32 dot-product error bound of
       the float64 oracle's (every token).
    2. The GPU's ids are a valid top-k of the float64 logits: bit-exact away
       from near-ties, any order consistent with the bound at a near-tie
       (routing_agreement).
    3. The oracle routes from the GPU's own logits ("given the same
       logits"): its ids must equal the GPU's bit for bit, its weights match
       within 1e-6, and the layer output y of every token (or of `tokens`)
       is compared with the oracle's eager expert loop on that routing.

    x, wr, bias: float64 inputs; expert_weights(e) -> float64 (w_gate_up[e],
    w_down[e]); shared: float64 shared-expert weights or None; y: device
    output.  Returns the oracle's (ids, w) from the GPU logits."""
    k, score = wl.k, wl.score
    g_logits = layer.logits.cpu().numpy().astype(np.float64)
    g_ids = layer.ids.cpu().numpy()
    g_w = layer.wts.cpu().numpy().astype(np.float64)
    L = O.router_logits(x, wr, bias)
    bound = O.logit_error_bound(x, wr, bias)
    assert (np.abs(g_logits - L) <= bound).all(), f"{what}: router logits outside the fp32 error bound"
    routing_agreement(g_ids, L, x, wr, bias, k)
    ids, w = O.route(g_logits, k, score)
    assert (ids == g_ids).all(), f"{what}: ids differ from the oracle's on the same logits"
    assert np.abs(g_w - w).max() <= 1e-6, f"{what}: routing weights"
    sel = np.arange(wl.T) if tokens is None else np.asarray(tokens)
    ref = O.moe_layer_eager(x[sel], ids[sel], w[sel], expert_weights, wl.E, shared)
    assert_close(host_values(y)[sel], ref, wl.dtype, f"{what} layer")
    return ids, w


@functools.lru_cache(maxsize=None)
def small_inputs(name: str):
    """All inputs of a small workload, in storage format and as float64."""
    wl = W.get(name)
    x = W.gen_x(wl)
    wr, bias = W.gen_router(wl)
    gu, dn = W.gen_all_experts(wl)
    sh = W.gen_shared(wl)
    return wl, dict(x=x, wr=wr, bias=bias, gu=gu, dn=dn, shared=sh)


def device_weights(wl, inp, device="cuda"):
    from mixture_experts_ffn_04_amd import MoeWeights
    dt = wl.dtype
    sh = inp["shared"]
    return MoeWeights(
        w_router=dev_tensor(inp["wr"], dt, device),
        bias=None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(device),
        w_gate_up=dev_tensor(inp["gu"], dt, device),
        w_down=dev_tensor(inp["dn"], dt, device),
        shared_gate_up=None if sh is None else dev_tensor(sh[0], dt, device),
        shared_down=None if sh is None else dev_tensor(sh[1], dt, device),
    )


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32
