"""Plant plausible mistakes in the CPU oracle (on the CPU, by monkeypatching)
and check that the pin suite catches every one of them."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import oracle_pins

_orig = {n: getattr(O, n) for n in dir(O) if callable(getattr(O, n))}


def _logits_no_bias(x, w_router, bias=None):
    return _orig["router_logits"](x, w_router, None)


def _logits_neg_bias(x, w_router, bias=None):
    return _orig["router_logits"](x, w_router, None if bias is None else -np.asarray(bias))


def _topk_high_index_ties(logits, k):
    L = np.asarray(logits, np.float64)[:, ::-1]
    return (L.shape[1] - 1 - _orig["select_topk"](L, k)).astype(np.int32)


def _topk_smallest(logits, k):
    return _orig["select_topk"](-np.asarray(logits, np.float64), k)


def _weights_not_renormalised(logits, ids, score):
    L = np.asarray(logits, np.float64)
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return np.take_along_axis(p, np.asarray(ids, np.int64), 1)


def _weights_sigmoid_as_softmax(logits, ids, score):
    return _orig["routing_weights"](logits, ids, "softmax")


def _permute_unstable(ids, E):
    counts, offsets, perm, inv = _orig["permute"](ids, E)
    perm = perm.copy()
    for e in range(E):
        perm[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return counts, offsets, perm, inv


def _permute_inclusive_offsets(ids, E):
    counts, offsets, perm, inv = _orig["permute"](ids, E)
    return counts, np.append(offsets[1:], offsets[-1]).astype(np.int32), perm, inv


def _gather_wrong_token(x, perm, k):
    return np.asarray(x, np.float64)[np.asarray(perm) % np.shape(x)[0]]


def _silu_sign(g):
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(g))


def _gate_up_swapped(xe, w):
    W = np.asarray(w, np.float64)
    f = W.shape[0] // 2
    return _orig["gate_up_swiglu"](xe, np.concatenate([W[f:], W[:f]], 0))


def _gate_used_twice(xe, w):
    W = np.asarray(w, np.float64)
    f = W.shape[0] // 2
    return _orig["gate_up_swiglu"](xe, np.concatenate([W[:f], W[:f]], 0))


def _down_not_transposed(he, w):
    return np.asarray(he, np.float64) @ np.asarray(w, np.float64)


def _combine_unweighted(y_perm, inv_perm, w, y_shared=None):
    return _orig["unpermute_combine"](y_perm, inv_perm, np.ones_like(np.asarray(w, np.float64)), y_shared)


def _combine_drops_shared(y_perm, inv_perm, w, y_shared=None):
    return _orig["unpermute_combine"](y_perm, inv_perm, w, None)


def _eager_wrong_slot_weight(x, ids, w, expert_weights, E, shared=None):
    w = np.asarray(w, np.float64)
    return _orig["moe_layer_eager"](x, ids, np.repeat(w[:, :1], w.shape[1], 1), expert_weights, E, shared)


def _eager_drops_shared(x, ids, w, expert_weights, E, shared=None):
    return _orig["moe_layer_eager"](x, ids, w, expert_weights, E, None)


def _route_decides_in_f64(logits, k, score, decide_dtype=np.float32):
    return _orig["route"](logits, k, score, np.float64)


def _bound_too_loose(x, w_router, bias=None):
    return 1000.0 * _orig["logit_error_bound"](x, w_router, bias)


def _bound_too_tight(x, w_router, bias=None):
    return 0.25 * _orig["logit_error_bound"](x, w_router, bias)


def _e2m1_bias0(code):
    v = _orig["e2m1_value"](code)
    return v if (int(code) >> 1) & 3 == 0 else 2.0 * v


def _e2m1_no_subnormal(code):
    code = int(code)
    if (code >> 1) & 3 == 0 and code & 1:
        return (-1.0 if code & 8 else 1.0) * 0.75
    return _orig["e2m1_value"](code)


def _e8m0_off_by_one(code):
    return _orig["e8m0_value"](code) / 2.0 if int(code) != 255 else float("nan")


def _mx_nibbles_swapped(q, scales):
    q = np.asarray(q, np.uint8)
    return _orig["mxfp4_dequantize"](((q & 0x0F) << 4) | (q >> 4), scales)


def _mx_block16(q, scales):
    v = _orig["mxfp4_dequantize"](q, np.repeat(np.asarray(scales, np.uint8), 1, axis=-1))
    s = np.asarray(scales, np.uint8)
    # scale of block b applied to elements [16b, 16b + 16)
    sv = np.array([_orig["e8m0_value"](c) for c in range(256)])[s]
    base = _orig["mxfp4_dequantize"](q, np.full_like(s, 127))
    K = base.shape[-1]
    idx = np.minimum(np.arange(K) // 16, s.shape[-1] - 1)
    return base * sv[..., idx]


MUTATIONS = {
    "logits drop bias": ("router_logits", _logits_no_bias),
    "logits bias sign": ("router_logits", _logits_neg_bias),
    "top-k ties to higher index": ("select_topk", _topk_high_index_ties),
    "top-k picks smallest": ("select_topk", _topk_smallest),
    "weights not renormalised": ("routing_weights", _weights_not_renormalised),
    "sigmoid scored as softmax": ("routing_weights", _weights_sigmoid_as_softmax),
    "route decides in float64": ("route", _route_decides_in_f64),
    "unstable group order": ("permute", _permute_unstable),
    "inclusive offsets": ("permute", _permute_inclusive_offsets),
    "gather wrong token": ("gather_rows", _gather_wrong_token),
    "silu sign": ("silu", _silu_sign),
    "gate/up swapped": ("gate_up_swiglu", _gate_up_swapped),
    "gate used twice": ("gate_up_swiglu", _gate_used_twice),
    "down not transposed": ("down", _down_not_transposed),
    "combine unweighted": ("unpermute_combine", _combine_unweighted),
    "combine drops shared": ("unpermute_combine", _combine_drops_shared),
    "eager wrong slot weight": ("moe_layer_eager", _eager_wrong_slot_weight),
    "eager drops shared": ("moe_layer_eager", _eager_drops_shared),
    "logit bound x1000": ("logit_error_bound", _bound_too_loose),
    "logit bound /4": ("logit_error_bound", _bound_too_tight),
    "e2m1 exponent bias 0": ("e2m1_value", _e2m1_bias0),
    "e2m1 subnormal as normal": ("e2m1_value", _e2m1_no_subnormal),
    "e8m0 bias 128": ("e8m0_value", _e8m0_off_by_one),
    "mxfp4 nibbles swapped": ("mxfp4_dequantize", _mx_nibbles_swapped),
    "mxfp4 blocks of 16": ("mxfp4_dequantize", _mx_block16),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:       # an assertion or a shape error both expose the mistake
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake: {name}"
