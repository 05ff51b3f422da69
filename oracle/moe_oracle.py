"""CPU oracle for the routed MoE feed-forward layer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding)
never calls it, and it shares no code with that path.

What it computes.  The article "Mixture of Experts (MoEs) in Transformers"
(Hugging Face blog), section "From Dense to Sparse": some dense
feed-forward blocks of a Transformer become a bank of experts -- each one a
small trainable network -- and a router chooses, per token and from that
token's activations, the few experts that will process it.  Section
"Expert Backend" lists the duties of any execution strategy (route each
token to the weights of its chosen experts, run their projections, scale by
the routing weights, and put the results back in token order) and three
interchangeable strategies: "eager" (iterate over the experts that received
tokens, running each expert's projections in turn; meant for checking and
debugging), "batched_mm" (copy the chosen weights per token and run one
batched matrix product) and "grouped_mm" (order the tokens by the expert
they were routed to, make each expert's tokens contiguous, run one grouped
matrix product).  All three evaluate the same sum

    y_t = sum_j  w_tj * FFN_{e_tj}(x_t)      (+ S(x_t) with a shared expert)

so this oracle is that definition written out in float64, structured like
the "eager" strategy, with the "grouped_mm" intermediates (counts, offsets,
permutation, per-row activations) exposed as well so every stage of the GPU
path can be checked on its own.

Readings taken where the pages are silent (each one is listed in the design
notes with its reason):
  * expert form: SwiGLU, FFN(x) = W_down (silu(W_gate x) * (W_up x)),
    silu(g) = g / (1 + exp(-g)); no biases.
  * packed layout: the "Dynamic Weight Loading with WeightConverter"
    subsection stacks the per-expert w1 (gate) and w3 (up) matrices along
    dim 0 and concatenates them along dim 1, and splits the packed down
    projection back into per-expert w2 matrices.  Per-expert matrices are
    [out, in], so w_gate_up is [E, 2f, d] with gate rows [0, f) and up rows
    [f, 2f), and w_down is [E, d, f].
  * router: logits = x W_r^T + bias; the k largest logits are selected in
    descending order, ties to the lower expert index; routing weights are a
    softmax over the k selected logits (identical to softmax-then-top-k with
    renormalisation) or, for the sigmoid router, sigmoid scores divided by
    their sum over the selection.  Selection is taken on the fp32 logit, the
    precision the GPU path decides in.
  * group order: the sort by expert ID is stable (ascending flat pair index
    p = t*k + j within an expert), so the permutation is unique.
  * the routing weight is applied after the down projection, in the combine;
    a shared expert (when present) is added unweighted.

Expert weights may also come in the MXFP4 format (OCP Microscaling
Formats Specification v1.0): mxfp4_dequantize gives their float64 values,
and the layer is then the same sum with those weights.

Every function below is pinned by CPU tests against something other than
itself: brute force on tiny inputs, closed forms, library routines
(numpy.argsort, torch.nn.functional) and invariants (weights sum to 1,
counts sum to T*k, token-permutation equivariance, one-hot router == dense
SwiGLU FFN, expert-partition sum).  No function is "parity unpinned".
"""
from __future__ import annotations

from typing import Callable, Optional

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


# ----------------------------------------------------------------- router

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """logits[t, e] = sum_i x[t, i] * w_router[e, i] + bias[e]   (float64).

    Every expert gets a score computed from the token's activations
    (article, section "From Dense to Sparse").
    """
    L = _f64(x) @ _f64(w_router).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    return L


def select_topk(logits, k: int) -> np.ndarray:
    """ids[t, j]: the j-th largest logit of row t; equal logits go to the lower
    expert index.  k rounds of "take the first maximum, then remove it".
    The comparison runs on the values as given (pass fp32 logits to decide in
    fp32)."""
    L = np.array(logits, dtype=F64, copy=True)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), np.int32)
    for j in range(k):
        a = np.argmax(L, axis=1)          # first occurrence of the maximum
        ids[:, j] = a
        L[np.arange(T), a] = -np.inf
    return ids


def routing_weights(logits, ids, score: str) -> np.ndarray:
    """w[t, j] for the selected experts (float64).

    softmax: exp(L_tj - m_t) / sum_j' exp(L_tj' - m_t), m_t = max_j L_tj
    sigmoid: s_tj / sum_j' s_tj',  s = 1 / (1 + exp(-L))
    """
    L = _f64(logits)
    sel = np.take_along_axis(L, np.asarray(ids, np.int64), axis=1)
    if score == "softmax":
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        return z / z.sum(axis=1, keepdims=True)
    if score == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-sel))
        return s / s.sum(axis=1, keepdims=True)
    raise ValueError(f"unknown score {score!r}")


def route(logits, k: int, score: str, decide_dtype=np.float32):
    """(ids, w): selection on logits rounded to `decide_dtype`, weights from
    the logits at full precision."""
    L = _f64(logits)
    ids = select_topk(L.astype(decide_dtype), k)
    return ids, routing_weights(L, ids, score)


# ----------------------------------------------------------- sort by expert

def permute(ids, E: int):
    """Order the routed pairs by expert ID and make each expert's pairs
    contiguous (the "grouped_mm" strategy, article section "Expert Backend").

    Returns
      counts[e]    number of pairs routed to expert e
      offsets[e]   first row of expert e's group; offsets[E] = T*k
      perm[r]      flat pair index p = t*k + j that lands on row r
      inv_perm[p]  row of pair p
    Within a group rows follow ascending p (stable order).
    """
    flat = np.asarray(ids, np.int64).ravel()
    P = flat.size
    counts = np.zeros(E, np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(P, np.int64)
    fill = offsets[:-1].copy()
    for p in range(P):                     # ascending p: stable
        e = flat[p]
        perm[fill[e]] = p
        fill[e] += 1
    inv_perm = np.empty(P, np.int64)
    inv_perm[perm] = np.arange(P)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv_perm.astype(np.int32))


def gather_rows(x, perm, k: int) -> np.ndarray:
    """x_perm[r] = x[perm[r] // k]: the token rows in grouped order."""
    return _f64(x)[np.asarray(perm, np.int64) // k]


# ------------------------------------------------------------------ experts

def silu(g):
    g = _f64(g)
    return g / (1.0 + np.exp(-g))


def gate_up_swiglu(xe, w_gate_up_e) -> np.ndarray:
    """h = silu(x W_gate^T) * (x W_up^T) for one expert; w_gate_up_e is
    [2f, d] with gate rows [0, f) and up rows [f, 2f)."""
    W = _f64(w_gate_up_e)
    f = W.shape[0] // 2
    xe = _f64(xe)
    return silu(xe @ W[:f].T) * (xe @ W[f:].T)


def down(he, w_down_e) -> np.ndarray:
    """y = h W_down^T for one expert; w_down_e is [d, f]."""
    return _f64(he) @ _f64(w_down_e).T


def expert_ffn(xe, w_gate_up_e, w_down_e) -> np.ndarray:
    return down(gate_up_swiglu(xe, w_gate_up_e), w_down_e)


def grouped_gate_up_swiglu(x_perm, w_gate_up, offsets) -> np.ndarray:
    """Per-expert loop over the grouped rows: H[R_e] = swiglu_e(X_perm[R_e])."""
    x_perm = _f64(x_perm)
    E = len(offsets) - 1
    f = np.shape(w_gate_up)[1] // 2
    H = np.zeros((x_perm.shape[0], f), F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            H[a:b] = gate_up_swiglu(x_perm[a:b], w_gate_up[e])
    return H


def grouped_down(h, w_down, offsets) -> np.ndarray:
    """Per-expert loop over the grouped rows: Y_perm[R_e] = H[R_e] W_down[e]^T."""
    h = _f64(h)
    E = len(offsets) - 1
    d = np.shape(w_down)[1]
    Y = np.zeros((h.shape[0], d), F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            Y[a:b] = down(h[a:b], w_down[e])
    return Y


def unpermute_combine(y_perm, inv_perm, w, y_shared=None) -> np.ndarray:
    """y[t] = sum_j w[t, j] * y_perm[inv_perm[t*k + j]]  (+ y_shared[t]);
    applies the routing weights, then collects the rows back in token order
    (article section "Expert Backend")."""
    w = _f64(w)
    T, k = w.shape
    rows = _f64(y_perm)[np.asarray(inv_perm, np.int64).reshape(T, k)]   # [T, k, d]
    y = np.zeros((T, rows.shape[2]), F64)
    for j in range(k):
        y += w[:, j:j + 1] * rows[:, j, :]
    if y_shared is not None:
        y += _f64(y_shared)
    return y


# ---------------------------------------------------------------- the layer

def moe_layer_eager(x, ids, w, expert_weights: Callable[[int], tuple], E: int,
                    shared=None) -> np.ndarray:
    """The "eager" strategy: loop over the experts that were selected, apply
    each expert's projections to its tokens, weight, and accumulate in token
    order.  `expert_weights(e)` returns (w_gate_up[e], w_down[e]) so that a
    large layer can be evaluated one expert at a time.  `shared` is
    (w_gate_up [1, 2f_s, d], w_down [1, d, f_s]) or None."""
    x = _f64(x)
    ids = np.asarray(ids, np.int64)
    w = _f64(w)
    T, k = ids.shape
    y = np.zeros((T, x.shape[1]), F64)
    for e in range(E):
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        gu, dn = expert_weights(e)
        ye = expert_ffn(x[t_idx], gu, dn)
        for n in range(t_idx.size):
            y[t_idx[n]] += w[t_idx[n], j_idx[n]] * ye[n]
    if shared is not None:
        y += expert_ffn(x, shared[0][0], shared[1][0])
    return y


def moe_layer_grouped(x, ids, w, w_gate_up, w_down, E: int, shared=None) -> dict:
    """The "grouped_mm" strategy written plainly, returning every stage:
    sort by expert, per-expert gate/up + SwiGLU, per-expert down, weighted
    combine back in token order."""
    T, k = np.shape(ids)
    counts, offsets, perm, inv_perm = permute(ids, E)
    x_perm = gather_rows(x, perm, k)
    H = grouped_gate_up_swiglu(x_perm, w_gate_up, offsets)
    Y_perm = grouped_down(H, w_down, offsets)
    y_shared = None
    if shared is not None:
        y_shared = expert_ffn(x, shared[0][0], shared[1][0])
    y = unpermute_combine(Y_perm, inv_perm, w, y_shared)
    return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv_perm,
                x_perm=x_perm, h=H, y_perm=Y_perm, y_shared=y_shared, y=y)


def moe_layer(x, w_router, bias, w_gate_up, w_down, k: int, score: str,
              shared=None) -> dict:
    """Router + eager expert loop for inputs that fit in memory."""
    L = router_logits(x, w_router, bias)
    ids, w = route(L, k, score)
    E = np.shape(w_router)[0]
    y = moe_layer_eager(x, ids, w, lambda e: (w_gate_up[e], w_down[e]), E, shared)
    return dict(logits=L, ids=ids, w=w, y=y)


# ------------------------------------------------------- mxfp4 expert weights

# The article's section "From Dense to Sparse" remarks that decoding would be
# faster still with kernels for the native mxfp4 format of the model's
# experts, and its section "Where Quantization Fits In" quantises weights per
# expert while they are loaded.  The format itself is the OCP Microscaling
# (MX) Formats Specification v1.0: an MXFP4 block holds 32 FP4 (E2M1)
# elements and one shared E8M0 scale; element i of a block stands for
# X * P_i, X = 2^(scale - 127) (scale code 255 is NaN), P_i the element's
# E2M1 value.
MX_BLOCK = 32


def e2m1_value(code: int) -> float:
    """The value of a 4-bit E2M1 element from its fields: sign bit 3,
    exponent bits 2..1 (bias 1), mantissa bit 0.  Exponent 0 is subnormal,
    0.M x 2^(1 - bias); otherwise 1.M x 2^(E - bias).  No Inf or NaN."""
    code = int(code)
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * (m * 0.5) * 2.0 ** (1 - 1)
    return sign * (1.0 + m * 0.5) * 2.0 ** (e - 1)


def e8m0_value(code: int) -> float:
    """An E8M0 scale: 2^(code - 127); code 255 is NaN."""
    code = int(code)
    return float("nan") if code == 255 else 2.0 ** (code - 127)


def mxfp4_dequantize(q, scales) -> np.ndarray:
    """float64 values of MXFP4 rows.

    q       [..., K/2] uint8: two elements per byte, element 2i in the low
            nibble and element 2i+1 in the high nibble (the byte order of the
            packed layout; the specification leaves packing open)
    scales  [..., K/32] uint8 E8M0 codes, one per block of 32 consecutive
            elements along the row
    """
    q = np.asarray(q, np.uint8)
    scales = np.asarray(scales, np.uint8)
    table = np.array([e2m1_value(c) for c in range(16)], F64)
    lo = table[q & 0x0F]
    hi = table[q >> 4]
    elems = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], q.shape[-1] * 2)
    K = elems.shape[-1]
    if scales.shape[-1] * MX_BLOCK != K:
        raise ValueError("one scale per 32 elements")
    sv = np.array([e8m0_value(c) for c in range(256)], F64)[scales]
    return (elems.reshape(*elems.shape[:-1], K // MX_BLOCK, MX_BLOCK) * sv[..., None]).reshape(elems.shape)


def topk_margin(logits, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit of each row (inf when
    k == E): how far the selection is from a tie."""
    L = np.sort(_f64(logits), axis=1)[:, ::-1]
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    return L[:, k - 1] - L[:, k]


def logit_error_bound(x, w_router, bias=None) -> np.ndarray:
    """Per-token bound on |fp32 logit - exact logit| for an fp32 dot product of
    length d accumulated in any order: gamma_d * sum_i |x_i w_i| (+|bias|)
    with gamma_d = d u / (1 - d u), u = 2^-24 (standard forward error bound
    for summation), plus the final rounding.  Returns [T, E]."""
    ax = np.abs(_f64(x))
    aw = np.abs(_f64(w_router))
    s = ax @ aw.T
    if bias is not None:
        s = s + np.abs(_f64(bias))[None, :]
    d = np.shape(x)[1]
    u = 2.0 ** -24
    g = (d + 2) * u / (1 - (d + 2) * u)
    return g * s + u * np.abs(_f64(x) @ _f64(w_router).T)
