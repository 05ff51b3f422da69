"""Seeded synthetic workloads for the routed MoE feed-forward layer.

This module only *makes inputs*: it draws seeded random tensors with the
shapes and value distributions of the five layer configurations and encodes
them in their storage format (bf16 bit patterns or fp32).  It holds none of
the layer's arithmetic (no router, no top-k, no sort, no projection), so both
the CPU oracle and the GPU path can take their inputs from here without
sharing any part of the method.

Workloads (shapes follow the article "Mixture of Experts (MoEs) in
Transformers", sections "From Dense to Sparse" and "Weight Loading Refactor":
gpt-oss-20b uses 4 of 32 experts, DeepSeek-V3 stores 256 experts per layer):

  c1      tiny fp32       T=64     d=128  f=256   E=8   k=2  softmax
  c2      Mixtral-shaped  T=4096   d=4096 f=14336 E=8   k=2  softmax
  c3_tN   gpt-oss-shaped  T=N      d=2880 f=2880  E=32  k=4  softmax  (decode)
  c4      fine-grained    T=8192   d=2048 f=768   E=128 k=8  softmax  Zipf(1.1)
  c5      DeepSeek-shaped T=16384  d=7168 f=2048  E=256 k=8  sigmoid  Zipf(1.0)
                                                        + shared expert f_s=2048
  c3mx_tN the gpt-oss-shaped decode layer with MXFP4 expert weights (the
          format gpt-oss ships its experts in; article section "From Dense
          to Sparse" remarks that native mxfp4 kernels would decode faster)

Storage layout (the packed per-layer expert tensors the article's weight
loading produces, see its "Dynamic Weight Loading with WeightConverter"
subsection):

  x          [T, d]          hidden states, ~N(0, 1)
  w_router   [E, d]          router projection, ~N(0, 0.02); the scaled-down shapes
                             use 0.02*sqrt(d_full/d) so their logits keep the
                             full-size spread against the Zipf bias
  bias       [E] fp32/None   router logit bias (Zipf popularity prior)
  w_gate_up  [E, 2f, d]      rows [0, f) = gate, rows [f, 2f) = up, ~N(0, 0.02)
  w_down     [E, d, f]       ~N(0, 0.02)
  shared     ([1, 2f_s, d], [1, d, f_s]) or None

Seeds: every tensor (and every expert of a packed tensor) has its own PCG64
stream keyed by (workload seed, tensor id, expert id), so any one expert can
be regenerated alone and experts can be generated in parallel threads.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# tensor ids for the seed key
_X, _WR, _BIASPERM, _WGU, _WD, _SGU, _SD, _LOGITS = 0, 1, 2, 3, 4, 5, 6, 7

WEIGHT_STD = 0.02


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    E: int
    k: int
    score: str            # "softmax" | "sigmoid"
    dtype: str            # "f32" | "bf16"
    zipf_s: Optional[float] = None
    f_shared: int = 0
    seed: int = 0
    router_std: float = 0.02   # scaled-down shapes raise it to keep the full-size logit spread
    experts: str = "dense"     # expert weight storage: "dense" (dtype) | "mxfp4"

    @property
    def P(self) -> int:
        """Routed (token, slot) pairs."""
        return self.T * self.k

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def expert_weight_bytes(self) -> float:
        """Bytes per expert weight element as stored (MXFP4: half a byte per
        element plus one scale byte per 32 elements)."""
        return 0.5 + 1.0 / 32 if self.experts == "mxfp4" else float(self.elem_bytes)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", 64, 128, 256, 8, 2, "softmax", "f32", seed=1),
    "c2": Workload("c2", 4096, 4096, 14336, 8, 2, "softmax", "bf16", seed=2),
    "c3_t1": Workload("c3_t1", 1, 2880, 2880, 32, 4, "softmax", "bf16", seed=31),
    "c3_t8": Workload("c3_t8", 8, 2880, 2880, 32, 4, "softmax", "bf16", seed=38),
    "c3_t32": Workload("c3_t32", 32, 2880, 2880, 32, 4, "softmax", "bf16", seed=332),
    "c3_t64": Workload("c3_t64", 64, 2880, 2880, 32, 4, "softmax", "bf16", seed=364),
    "c3mx_t1": Workload("c3mx_t1", 1, 2880, 2880, 32, 4, "softmax", "bf16", seed=41, experts="mxfp4"),
    "c3mx_t8": Workload("c3mx_t8", 8, 2880, 2880, 32, 4, "softmax", "bf16", seed=48, experts="mxfp4"),
    "c3mx_t32": Workload("c3mx_t32", 32, 2880, 2880, 32, 4, "softmax", "bf16", seed=432, experts="mxfp4"),
    "c3mx_t64": Workload("c3mx_t64", 64, 2880, 2880, 32, 4, "softmax", "bf16", seed=464, experts="mxfp4"),
    "c4": Workload("c4", 8192, 2048, 768, 128, 8, "softmax", "bf16", zipf_s=1.1, seed=4),
    "c5": Workload("c5", 16384, 7168, 2048, 256, 8, "sigmoid", "bf16", zipf_s=1.0,
                   f_shared=2048, seed=5),
}

# Scaled-down shapes of the same families: small enough for the oracle to
# finish in seconds, large enough to span several GEMM tiles and leave a
# ragged tail in every tiled dimension that the layer allows to be ragged
# (T and the per-expert row counts).
SMALL_WORKLOADS = {
    "c1": WORKLOADS["c1"],
    "c2s": Workload("c2s", 333, 512, 768, 8, 2, "softmax", "bf16", seed=102,
                    router_std=0.02 * (4096 / 512) ** 0.5),
    "c3s_t1": Workload("c3s_t1", 1, 576, 640, 32, 4, "softmax", "bf16", seed=131,
                       router_std=0.02 * (2880 / 576) ** 0.5),
    "c3s_t37": Workload("c3s_t37", 37, 576, 640, 32, 4, "softmax", "bf16", seed=137,
                        router_std=0.02 * (2880 / 576) ** 0.5),
    "c3mxs_t1": Workload("c3mxs_t1", 1, 576, 640, 32, 4, "softmax", "bf16", seed=141,
                         router_std=0.02 * (2880 / 576) ** 0.5, experts="mxfp4"),
    "c3mxs_t37": Workload("c3mxs_t37", 37, 576, 640, 32, 4, "softmax", "bf16", seed=147,
                          router_std=0.02 * (2880 / 576) ** 0.5, experts="mxfp4"),
    # the same layer at d = 1536, f = 1344 (a K that ends in half a
    # 128-element MXFP4 quad, and 21 column blocks of 64), 37 tokens
    "c3mxm_t37": Workload("c3mxm_t37", 37, 1536, 1344, 32, 4, "softmax", "bf16", seed=157,
                          router_std=0.02 * (2880 / 1536) ** 0.5, experts="mxfp4"),
    "c4s": Workload("c4s", 517, 256, 192, 128, 8, "softmax", "bf16", zipf_s=1.1, seed=104,
                    router_std=0.02 * (2048 / 256) ** 0.5),
    "c5s": Workload("c5s", 301, 448, 128, 256, 8, "sigmoid", "bf16", zipf_s=1.0,
                    f_shared=192, seed=105, router_std=0.02 * (7168 / 448) ** 0.5),
}


def get(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    return SMALL_WORKLOADS[name]


# ---------------------------------------------------------------- encodings

def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite normal random draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    tmp = np.right_shift(u, 16)
    np.bitwise_and(tmp, 1, out=tmp)
    tmp += np.uint32(0x7FFF)
    tmp += u
    tmp >>= 16
    return tmp.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the exact fp32 values they encode."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def values(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> the exact values it encodes, as float64."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _encode(a32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, np.float32)


def _rng(wl: Workload, tensor: int, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng([wl.seed, tensor, idx])


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


# ---------------------------------------------------------------- tensors

def gen_x(wl: Workload, T: Optional[int] = None) -> np.ndarray:
    """Hidden states [T, d] ~ N(0, 1) in storage format."""
    T = wl.T if T is None else T
    return _encode(_normal(_rng(wl, _X), (T, wl.d), 1.0), wl.dtype)


def gen_router(wl: Workload):
    """(w_router [E, d] in storage format, bias [E] fp32 or None).

    With a Zipf exponent s, expert e gets the log-prior bias ln p_r with
    p_r = r^-s / sum_{r'=1..E} r'^-s, where r = rank(e) is a seeded
    permutation of 1..E.  This skews expert popularity toward a Zipf law
    (the realised load is reported, not tuned).
    """
    w = _encode(_normal(_rng(wl, _WR), (wl.E, wl.d), wl.router_std), wl.dtype)
    if wl.zipf_s is None:
        return w, None
    ranks = _rng(wl, _BIASPERM).permutation(wl.E) + 1
    r = np.arange(1, wl.E + 1, dtype=np.float64)
    p = r ** (-wl.zipf_s)
    p /= p.sum()
    bias = np.log(p[ranks - 1]).astype(np.float32)
    return w, bias


def gen_expert(wl: Workload, e: int):
    """(w_gate_up[e] [2f, d], w_down[e] [d, f]) in storage format."""
    gu = _encode(_normal(_rng(wl, _WGU, e), (2 * wl.f, wl.d), WEIGHT_STD), wl.dtype)
    dn = _encode(_normal(_rng(wl, _WD, e), (wl.d, wl.f), WEIGHT_STD), wl.dtype)
    return gu, dn


# MXFP4 scale codes are drawn from MX_SCALE_CODE + {-1, 0, 1}: with codes
# uniform over the 16 E2M1 values (root mean square 2.93), 2^(120 - 127)
# gives an element spread of about 0.023, close to the dense weights' 0.02.
MX_SCALE_CODE = 120


def _mx_rows(rng: np.random.Generator, rows: int, K: int):
    """Random MXFP4 rows: codes [rows, K/2] uint8 (two E2M1 codes per byte,
    every code equally likely) and E8M0 scale codes [rows, K/32] uint8."""
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = (MX_SCALE_CODE + rng.integers(-1, 2, size=(rows, K // 32))).astype(np.uint8)
    return q, s


def gen_expert_mxfp4(wl: Workload, e: int):
    """MXFP4 storage of expert e: (gate_up codes [2f, d/2], gate_up scales
    [2f, d/32], down codes [d, f/2], down scales [d, f/32]); the blocks of
    32 run along each row's input dimension (d for gate/up, f for down)."""
    gq, gs = _mx_rows(_rng(wl, _WGU, e), 2 * wl.f, wl.d)
    dq, ds = _mx_rows(_rng(wl, _WD, e), wl.d, wl.f)
    return gq, gs, dq, ds


def gen_all_experts_mxfp4(wl: Workload):
    """Packed MXFP4 experts: codes and scales stacked over the experts."""
    parts = [gen_expert_mxfp4(wl, e) for e in range(wl.E)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(4))


def gen_shared(wl: Workload):
    """Shared expert ([1, 2f_s, d], [1, d, f_s]) in storage format, or None."""
    if not wl.f_shared:
        return None
    fs = wl.f_shared
    gu = _encode(_normal(_rng(wl, _SGU), (1, 2 * fs, wl.d), WEIGHT_STD), wl.dtype)
    dn = _encode(_normal(_rng(wl, _SD), (1, wl.d, fs), WEIGHT_STD), wl.dtype)
    return gu, dn


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def iter_experts(wl: Workload, experts=None, threads: Optional[int] = None):
    """Yield (e, w_gate_up[e], w_down[e]) in expert order, generated in a
    thread pool (numpy's generators release the GIL while filling)."""
    experts = list(range(wl.E)) if experts is None else list(experts)
    threads = threads or default_threads()
    with ThreadPoolExecutor(threads) as ex:
        window = 2 * threads
        futs = {}
        for i, e in enumerate(experts):
            futs[i] = ex.submit(gen_expert, wl, e)
            if i >= window:
                j = i - window
                yield (experts[j],) + futs.pop(j).result()
        for j in sorted(futs):
            yield (experts[j],) + futs[j].result()


def gen_all_experts(wl: Workload, threads: Optional[int] = None):
    """Packed (w_gate_up [E, 2f, d], w_down [E, d, f]) in storage format."""
    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    gu = np.empty((wl.E, 2 * wl.f, wl.d), sdt)
    dn = np.empty((wl.E, wl.d, wl.f), sdt)
    for e, g, w in iter_experts(wl, threads=threads):
        gu[e] = g
        dn[e] = w
    return gu, dn


# ---------------------------------------------------------------- test data

def gen_tied_logits(T: int, E: int, seed: int, levels: int = 6) -> np.ndarray:
    """fp32 logits [T, E] drawn from a few discrete levels, so that most rows
    hold exact ties (for checking the lowest-index tie rule bit-exactly)."""
    rng = np.random.default_rng([seed, _LOGITS])
    lv = rng.integers(0, levels, size=(T, E)).astype(np.float32)
    return (lv * np.float32(0.5) - np.float32(1.0)).astype(np.float32)


def gen_logits(T: int, E: int, seed: int, std: float = 1.5) -> np.ndarray:
    """Continuous fp32 logits [T, E] ~ N(0, std)."""
    rng = np.random.default_rng([seed, _LOGITS, 1])
    return _normal(rng, (T, E), std)


def gen_ids(T: int, E: int, k: int, seed: int, zipf_s: Optional[float] = None) -> np.ndarray:
    """A valid routing table [T, k] int32: k distinct experts per token,
    drawn uniformly or with Zipf popularity (for permutation tests that do
    not go through the router)."""
    rng = np.random.default_rng([seed, _LOGITS, 2])
    if zipf_s is None:
        p = np.full(E, 1.0 / E)
    else:
        p = np.arange(1, E + 1, dtype=np.float64) ** (-zipf_s)
        p /= p.sum()
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False, p=p)
    return out


def gen_matrix(shape, seed: int, std: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """A seeded ~N(0, std) array in storage format (stand-alone inputs for
    testing one stage of the layer, e.g. activations fed to the down
    projection or expert outputs fed to the combine)."""
    rng = np.random.default_rng([seed, _LOGITS, 3])
    return _encode(_normal(rng, tuple(shape), std), dtype)
