"""Pins for the CPU oracle: checks against things other than the oracle
itself (brute force, closed forms, library routines, invariants).

Each pin is a plain function that raises AssertionError on failure, so the
same set can be run as tests (test_oracle_pins.py) and re-run against an
oracle with a planted mistake (test_oracle_mutations.py) to show that each
plausible mistake is caught by at least one pin.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import moe_workloads as W
from oracle import moe_oracle as O


def _rng(seed):
    return np.random.default_rng([777, seed])


def _tiny_layer(seed, T=13, d=16, f=24, E=6, k=2, shared_fs=0):
    """Random tiny layer in float64, packed the way the article's weight
    converter packs it: w1 (gate) and w3 (up) per expert are [f, d]; the
    experts are stacked on dim 0, then the two stacks are concatenated on
    dim 1; w2 (down) per expert is [d, f], stacked on dim 0."""
    r = _rng(seed)
    x = r.standard_normal((T, d))
    w1 = [r.standard_normal((f, d)) * 0.3 for _ in range(E)]
    w3 = [r.standard_normal((f, d)) * 0.3 for _ in range(E)]
    w2 = [r.standard_normal((d, f)) * 0.3 for _ in range(E)]
    gate_up = torch.cat([torch.stack([torch.from_numpy(a) for a in w1]),
                         torch.stack([torch.from_numpy(a) for a in w3])], dim=1).numpy()
    down = torch.stack([torch.from_numpy(a) for a in w2]).numpy()
    wr = r.standard_normal((E, d)) * 0.5
    bias = r.standard_normal(E) * 0.1
    shared = None
    if shared_fs:
        sg = r.standard_normal((shared_fs, d)) * 0.3
        su = r.standard_normal((shared_fs, d)) * 0.3
        sd = r.standard_normal((d, shared_fs)) * 0.3
        shared = (np.concatenate([sg, su], 0)[None], sd[None], (sg, su, sd))
    return dict(x=x, w1=w1, w3=w3, w2=w2, gate_up=gate_up, down=down, wr=wr,
                bias=bias, shared=shared, T=T, d=d, f=f, E=E, k=k)


def _dense_swiglu(x, wg, wu, wd):
    """Textbook SwiGLU FFN with torch.nn.functional (float64)."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    h = F.silu(F.linear(X, torch.from_numpy(wg))) * F.linear(X, torch.from_numpy(wu))
    return F.linear(h, torch.from_numpy(wd)).numpy()


def _batched_mm_layer(x, ids, w, gate_up, down, shared=None):
    """The article's "batched_mm" formulation: per token, gather the
    selected experts' weights and run one batched GEMM (torch.bmm, float64)."""
    X = torch.from_numpy(np.asarray(x, np.float64))
    GU = torch.from_numpy(np.asarray(gate_up, np.float64))
    DN = torch.from_numpy(np.asarray(down, np.float64))
    idx = torch.from_numpy(np.asarray(ids, np.int64))
    T, k = idx.shape
    f = GU.shape[1] // 2
    gu = GU[idx.reshape(-1)]                                   # [T*k, 2f, d]
    xr = X.repeat_interleave(k, dim=0).unsqueeze(2)            # [T*k, d, 1]
    a = torch.bmm(gu, xr).squeeze(2)                           # [T*k, 2f]
    h = F.silu(a[:, :f]) * a[:, f:]
    yk = torch.bmm(DN[idx.reshape(-1)], h.unsqueeze(2)).squeeze(2)   # [T*k, d]
    y = (yk.reshape(T, k, -1) * torch.from_numpy(np.asarray(w, np.float64)).unsqueeze(2)).sum(1)
    if shared is not None:
        sg, su, sd = shared
        y = y + torch.from_numpy(_dense_swiglu(x, sg, su, sd))
    return y.numpy()


# ------------------------------------------------------------------ router

def pin_logits_library():
    L = _tiny_layer(1)
    ref = F.linear(torch.from_numpy(L["x"]), torch.from_numpy(L["wr"]),
                   torch.from_numpy(L["bias"])).numpy()
    got = O.router_logits(L["x"], L["wr"], L["bias"])
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    ref0 = F.linear(torch.from_numpy(L["x"]), torch.from_numpy(L["wr"])).numpy()
    np.testing.assert_allclose(O.router_logits(L["x"], L["wr"], None), ref0, rtol=1e-13, atol=1e-13)


def _brute_topk(row, k):
    return sorted(range(len(row)), key=lambda e: (-row[e], e))[:k]


def pin_topk_bruteforce():
    for seed, (T, E, k) in enumerate([(40, 8, 2), (30, 32, 4), (20, 128, 8), (10, 256, 8), (9, 5, 5)]):
        for Lg in (W.gen_logits(T, E, seed), W.gen_tied_logits(T, E, seed, levels=3)):
            ids = O.select_topk(Lg, k)
            for t in range(T):
                assert list(ids[t]) == _brute_topk(list(Lg[t]), k), (T, E, k, t)


def pin_topk_closed_forms():
    for E, k in [(8, 2), (32, 4), (256, 8), (7, 7)]:
        ids = O.select_topk(np.zeros((3, E), np.float32), k)
        assert (ids == np.arange(k)[None]).all()                  # all equal -> lowest indices
    row = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5]], np.float32)
    assert list(O.select_topk(row, 4)[0]) == [1, 2, 4, 0]
    row = np.array([[3.0, -2.0, 7.0, 1.0]])
    assert list(O.select_topk(row, 4)[0]) == [2, 0, 3, 1]         # k = E: full order


def pin_weights_closed_forms():
    # sum to one
    Lg = W.gen_logits(50, 16, 3).astype(np.float64)
    for score in ("softmax", "sigmoid"):
        for k in (1, 2, 4, 8):
            ids = O.select_topk(Lg, k)
            w = O.routing_weights(Lg, ids, score)
            assert np.all(np.abs(w.sum(1) - 1) <= 1e-12)
            assert np.all(w > 0)
            if k == 1:
                assert np.all(w == 1.0)
    # softmax with two selected: w0 = 1 / (1 + e^(L1 - L0)); L = [ln 3, 0] -> [3/4, 1/4]
    row = np.array([[math.log(3.0), 0.0, -5.0]])
    w = O.routing_weights(row, O.select_topk(row, 2), "softmax")
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=0, atol=1e-15)
    # sigmoid: sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4 -> normalised [3/4, 1/4]
    row = np.array([[math.log(3.0), -math.log(3.0), -9.0]])
    w = O.routing_weights(row, O.select_topk(row, 2), "sigmoid")
    np.testing.assert_allclose(w[0], [0.75, 0.25], rtol=0, atol=1e-15)
    # sigmoid ratio is NOT the softmax ratio: sigma(2)/sigma(0) != e^2
    row = np.array([[2.0, 0.0]])
    ws = O.routing_weights(row, O.select_topk(row, 2), "sigmoid")
    s2 = 1 / (1 + math.exp(-2.0))
    np.testing.assert_allclose(ws[0], [s2 / (s2 + 0.5), 0.5 / (s2 + 0.5)], rtol=1e-15)
    # all equal logits -> exactly 1/k
    for k in (1, 2, 4, 8):
        row = np.full((2, 8), 0.25)
        for score in ("softmax", "sigmoid"):
            w = O.routing_weights(row, O.select_topk(row, k), score)
            assert np.all(w == 1.0 / k)


def pin_weights_library():
    """softmax over all E, take the top k, renormalise (torch.softmax) ==
    softmax over the selected logits; sigmoid scores via torch.sigmoid."""
    Lg = W.gen_logits(40, 32, 5).astype(np.float64)
    k = 4
    ids = O.select_topk(Lg, k)
    p = torch.softmax(torch.from_numpy(Lg), dim=1).numpy()
    sel = np.take_along_axis(p, ids.astype(np.int64), 1)
    np.testing.assert_allclose(O.routing_weights(Lg, ids, "softmax"), sel / sel.sum(1, keepdims=True),
                               rtol=1e-13)
    s = torch.sigmoid(torch.from_numpy(Lg)).numpy()
    sel = np.take_along_axis(s, ids.astype(np.int64), 1)
    np.testing.assert_allclose(O.routing_weights(Lg, ids, "sigmoid"), sel / sel.sum(1, keepdims=True),
                               rtol=1e-13)
    # the top-k of torch.topk on distinct values matches (values sorted descending)
    tv, ti = torch.topk(torch.from_numpy(Lg), k, dim=1)
    assert (ti.numpy() == ids).all()


def pin_route_decides_in_fp32():
    """Two logits that differ only below fp32 resolution are a tie in fp32:
    the lower index wins even though its float64 value is smaller."""
    row = np.array([[1.0, 1.0 + 1e-12, 0.0]])
    ids, w = O.route(row, 1, "softmax")
    assert ids[0, 0] == 0
    ids64 = O.select_topk(row, 1)
    assert ids64[0, 0] == 1


# ---------------------------------------------------------------- permute

def pin_permute_library():
    cases = [(50, 8, 2, None), (37, 32, 4, None), (64, 128, 8, 1.1), (33, 256, 8, 1.0), (1, 4, 4, None)]
    for seed, (T, E, k, s) in enumerate(cases):
        ids = W.gen_ids(T, E, k, seed, s)
        counts, offsets, perm, inv = O.permute(ids, E)
        flat = ids.ravel()
        assert (perm == np.argsort(flat, kind="stable")).all()
        assert (counts == np.bincount(flat, minlength=E)).all()
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert (np.diff(offsets) == counts).all()
        assert (inv[perm] == np.arange(T * k)).all()
        assert (np.sort(perm) == np.arange(T * k)).all()
        assert (np.diff(flat[perm]) >= 0).all()
        for e in range(E):
            g = perm[offsets[e]:offsets[e + 1]]
            assert (flat[g] == e).all() and (np.diff(g) > 0).all()


def pin_gather_rows():
    x = _rng(9).standard_normal((7, 5))
    perm = np.array([3, 0, 13, 6, 1, 10, 2, 4, 5, 7, 8, 9, 11, 12])
    got = O.gather_rows(x, perm, 2)
    for r, p in enumerate(perm):
        assert (got[r] == x[p // 2]).all()


# ---------------------------------------------------------------- experts

def pin_silu():
    assert O.silu(0.0) == 0.0
    np.testing.assert_allclose(O.silu(1.0), 1.0 / (1.0 + math.exp(-1.0)), rtol=1e-15)
    np.testing.assert_allclose(O.silu(1.0), 0.7310585786300049, rtol=1e-15)
    g = np.linspace(-8, 8, 101)
    np.testing.assert_allclose(O.silu(g) - O.silu(-g), g, atol=1e-14)     # silu(g) - silu(-g) = g
    np.testing.assert_allclose(O.silu(g), F.silu(torch.from_numpy(g)).numpy(), rtol=1e-14, atol=1e-15)
    assert abs(O.silu(40.0) - 40.0) < 1e-12 and abs(O.silu(-40.0)) < 1e-15


def pin_expert_dense():
    """One expert == textbook dense SwiGLU FFN; a square case (d == f) makes
    a transposed operand a numeric, not a shape, error."""
    for (d, f) in [(16, 24), (20, 20)]:
        L = _tiny_layer(11, d=d, f=f)
        for e in (0, 3):
            ref = _dense_swiglu(L["x"], L["w1"][e], L["w3"][e], L["w2"][e])
            got = O.expert_ffn(L["x"], L["gate_up"][e], L["down"][e])
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_one_hot_router_is_dense():
    """k = 1 (weight exactly 1) and a router that sends every token to expert
    e reproduces the dense SwiGLU FFN of expert e; so does k = 2 when the
    second logit is 800 below (its softmax weight underflows to 0)."""
    L = _tiny_layer(12, E=5, d=20, f=20)
    for e in range(L["E"]):
        wr = np.zeros((L["E"], L["d"]))
        bias = np.zeros(L["E"])
        bias[e] = 1000.0
        bias[(e + 1) % L["E"]] = 200.0
        ref = _dense_swiglu(L["x"], L["w1"][e], L["w3"][e], L["w2"][e])
        for k in (1, 2):
            out = O.moe_layer(L["x"], wr, bias, L["gate_up"], L["down"], k, "softmax")
            assert (out["ids"][:, 0] == e).all()
            assert (out["w"][:, 0] == 1.0).all()
            np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-12)


def pin_identical_experts_are_dense():
    """If all experts are the same FFN the routing weights sum to 1, so the
    layer equals that dense FFN whatever the routing (both scores)."""
    L = _tiny_layer(13, E=6, k=3)
    E = L["E"]
    gu = np.repeat(L["gate_up"][:1], E, 0)
    dn = np.repeat(L["down"][:1], E, 0)
    ref = _dense_swiglu(L["x"], L["w1"][0], L["w3"][0], L["w2"][0])
    for score in ("softmax", "sigmoid"):
        out = O.moe_layer(L["x"], L["wr"], L["bias"], gu, dn, 3, score)
        np.testing.assert_allclose(out["y"], ref, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------- layer

def pin_layer_three_strategies():
    """eager loop == grouped (sort / group / per-group GEMM / combine) ==
    batched_mm (per-token gathered weights, torch.bmm), with and without a
    shared expert and for both scores."""
    for seed, (T, d, f, E, k, fs, score) in enumerate([
            (17, 16, 24, 6, 2, 0, "softmax"), (23, 12, 12, 8, 3, 0, "sigmoid"),
            (11, 16, 8, 16, 8, 10, "sigmoid"), (9, 8, 16, 4, 4, 0, "softmax")]):
        L = _tiny_layer(20 + seed, T=T, d=d, f=f, E=E, k=k, shared_fs=fs)
        logits = O.router_logits(L["x"], L["wr"], L["bias"])
        ids, w = O.route(logits, k, score)
        shared = None if not fs else L["shared"][:2]
        eager = O.moe_layer_eager(L["x"], ids, w, lambda e: (L["gate_up"][e], L["down"][e]), E, shared)
        grouped = O.moe_layer_grouped(L["x"], ids, w, L["gate_up"], L["down"], E, shared)
        bmm = _batched_mm_layer(L["x"], ids, w, L["gate_up"], L["down"],
                                None if not fs else L["shared"][2])
        np.testing.assert_allclose(eager, bmm, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(grouped["y"], bmm, rtol=1e-12, atol=1e-12)


def pin_layer_closed_forms():
    L = _tiny_layer(30, shared_fs=8)
    x, E, k = L["x"], L["E"], L["k"]
    shared = L["shared"][:2]
    out = O.moe_layer(x, L["wr"], L["bias"], L["gate_up"], L["down"], k, "sigmoid", shared)
    # W_down = 0 -> only the shared expert remains
    y0 = O.moe_layer(x, L["wr"], L["bias"], L["gate_up"], 0 * L["down"], k, "sigmoid", shared)["y"]
    np.testing.assert_allclose(y0, _dense_swiglu(x, *L["shared"][2]), rtol=1e-12, atol=1e-12)
    # doubling W_down doubles the routed part exactly
    y1 = O.moe_layer(x, L["wr"], L["bias"], L["gate_up"], L["down"], k, "sigmoid")["y"]
    y2 = O.moe_layer(x, L["wr"], L["bias"], L["gate_up"], 2 * L["down"], k, "sigmoid")["y"]
    assert (y2 == 2 * y1).all()
    # x = 0 -> y = 0
    z = O.moe_layer(0 * x, L["wr"], L["bias"], L["gate_up"], L["down"], k, "softmax", shared)["y"]
    assert (z == 0).all()
    assert np.isfinite(out["y"]).all()


def pin_token_permutation_equivariance():
    L = _tiny_layer(31, T=29, E=8, k=2)
    pi = _rng(5).permutation(L["T"])
    a = O.moe_layer(L["x"], L["wr"], L["bias"], L["gate_up"], L["down"], 2, "softmax")
    b = O.moe_layer(L["x"][pi], L["wr"], L["bias"], L["gate_up"], L["down"], 2, "softmax")
    assert (b["ids"] == a["ids"][pi]).all()
    np.testing.assert_allclose(b["y"], a["y"][pi], rtol=1e-13, atol=1e-14)


def pin_expert_partition_sum():
    """Sum over a partition of the experts of the outputs restricted to each
    part (non-local experts masked out, as an expert-parallel shard does)
    equals the full output."""
    L = _tiny_layer(32, T=21, E=8, k=3)
    logits = O.router_logits(L["x"], L["wr"], L["bias"])
    ids, w = O.route(logits, 3, "softmax")
    full = O.moe_layer_eager(L["x"], ids, w, lambda e: (L["gate_up"][e], L["down"][e]), 8)
    acc = np.zeros_like(full)
    for part in ([0, 1, 2], [3, 4], [5, 6, 7]):
        wm = np.where(np.isin(ids, part), w, 0.0)
        acc += O.moe_layer_eager(L["x"], ids, wm, lambda e: (L["gate_up"][e], L["down"][e]), 8)
    np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-13)


def pin_combine():
    y_perm = _rng(40).standard_normal((6, 3))
    inv = np.array([4, 0, 2, 5, 1, 3])
    w = np.array([[0.25, 0.75], [1.0, 0.0], [0.5, 0.5]])
    ys = _rng(41).standard_normal((3, 3))
    got = O.unpermute_combine(y_perm, inv, w, ys)
    ref = np.stack([0.25 * y_perm[4] + 0.75 * y_perm[0], y_perm[2], 0.5 * y_perm[1] + 0.5 * y_perm[3]]) + ys
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=1e-15)


def pin_margin_and_error_bound():
    Lg = np.array([[1.0, 3.0, 2.0, 2.5]])
    assert O.topk_margin(Lg, 2)[0] == 0.5 and O.topk_margin(Lg, 4)[0] == np.inf
    wl = W.get("c4s")
    x = W.values(W.gen_x(wl), wl.dtype)
    wr, bias = W.gen_router(wl)
    wr = W.values(wr, wl.dtype)
    exact = O.router_logits(x, wr, bias)
    f32 = (x.astype(np.float32) @ wr.astype(np.float32).T + bias[None]).astype(np.float64)
    assert (np.abs(f32 - exact) <= O.logit_error_bound(x, wr, bias)).all()


def pin_logit_error_bound_is_attained():
    """The logit bound is the worst-case error of an fp32 dot product summed
    in any order, so some order must come close to it.  Sum 1 and then d-1
    products of exactly 2^-24 (x = w = 2^-12) one by one in fp32: every
    partial sum lies exactly halfway between 1 and the next fp32 number above
    it, and the tie goes to the even neighbour, 1.0, so every step rounds
    down and the error is (d-1) 2^-24 against an exact sum of 1 + (d-1) 2^-24.
    The bound must cover that error (lower side) and exceed it by under 10%
    (upper side: a looser bound would accept wrong GPU logits and excuse
    routing differences that are not near-ties)."""
    for d in (64, 256, 1024, 4096):
        x = np.full((1, d), 2.0 ** -12)
        w = np.full((1, d), 2.0 ** -12)
        x[0, 0] = w[0, 0] = 1.0
        acc = np.float32(0.0)
        for i in range(d):
            acc = np.float32(acc + np.float32(x[0, i]) * np.float32(w[0, i]))
        exact = 1.0 + (d - 1) * 2.0 ** -24
        err = abs(float(acc) - exact)
        assert float(acc) == 1.0 and err == (d - 1) * 2.0 ** -24
        b = O.logit_error_bound(x, w)[0, 0]
        assert err <= b <= 1.1 * err, (d, err, b)


# ------------------------------------------------------------- mxfp4 weights

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def pin_mxfp4_element_table():
    """The 16 E2M1 codes decode to the table of the OCP MX specification
    (tests/golden/mxfp4_e2m1_values.json), signed zero included."""
    import json
    ref = json.load(open(__import__("os").path.join(GOLDEN, "mxfp4_e2m1_values.json")))["values"]
    for c in range(16):
        v = O.e2m1_value(c)
        assert v == ref[c] and math.copysign(1.0, v) == math.copysign(1.0, ref[c]), (c, v, ref[c])


def pin_mxfp4_scale_library():
    """E8M0 scale codes against torch's float8_e8m0fnu decoding (every code:
    powers of two 2^-127 .. 2^127, and NaN for 255)."""
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = np.array([O.e8m0_value(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert (got[:255] == ref[:255]).all()


def pin_mxfp4_dequantize_layout():
    """Closed forms of the packed layout: element 2i in the low nibble, one
    scale per 32 consecutive elements along the row."""
    q = np.zeros((2, 32), np.uint8)              # 2 rows of 64 elements
    q[0, 0], q[0, 1] = 0x21, 0xF7                # 0.5, 1.0, 6, -6
    q[0, 15] = 0x20                              # element 31 (last of block 0): 1.0
    q[1, 16] = 0x3A                              # element 32: -1.0, element 33: 1.5
    s = np.array([[128, 120], [127, 130]], np.uint8)
    v = O.mxfp4_dequantize(q, s)
    assert v.shape == (2, 64)
    assert list(v[0, :4]) == [1.0, 2.0, 12.0, -12.0]        # x 2^(128-127)
    assert v[0, 31] == 2.0                                    # still block 0's scale
    assert (v[0, 4:31] == 0).all() and (v[0, 32:] == 0).all()
    assert list(v[1, 32:34]) == [-8.0, 12.0]                  # second block x 2^(130-127)
    assert (v[1, :32] == 0).all() and (v[1, 34:] == 0).all()
    # every code in every nibble position, scale 1: the element table in order
    q = np.arange(256, dtype=np.uint8).reshape(8, 32)
    v = O.mxfp4_dequantize(q, np.full((8, 2), 127, np.uint8)).reshape(-1)
    table = [O.e2m1_value(c) for c in range(16)]
    assert all(v[2 * b] == table[b & 15] and v[2 * b + 1] == table[b >> 4] for b in range(256))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
