"""Thin Python binding over the libmoe C ABI (include/libmoe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of libmoe.so.  PyTorch supplies device memory and the current HIP stream.
There is no fallback: if libmoe.so is missing or no GPU is present the calls
raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

from .placement import expert_map

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1

EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_route", "moe_topk",
    "moe_permute_workspace_size", "moe_permute", "moe_grouped_gemm_gateup_swiglu",
    "moe_grouped_gemm_down", "moe_unpermute_combine", "moe_decode_gateup_swiglu",
    "moe_decode_down", "moe_decode_gateup_swiglu_gather", "moe_grouped_gemm_gateup_swiglu_gather",
    "moe_localize_ids", "moe_localize_ids_strided", "moe_localize_ids_mapped", "moe_permute_noalloc", "moe_batched_gateup_swiglu",
    "moe_batched_down_combine",
    "moe_decode_gateup_swiglu_mxfp4", "moe_decode_down_mxfp4", "moe_batched_gateup_swiglu_mxfp4",
    "moe_batched_down_combine_mxfp4", "moe_batched_gateup_swiglu_select", "moe_batched_gateup_swiglu_mxfp4_select",
)

_lib: Optional[ctypes.CDLL] = None

P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t

_SIGS = {
    "moe_abi_version": ([], ctypes.c_int),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_route": ([P, P, P, I64, I64, I32, I32, ctypes.c_int, ctypes.c_int, P, P, P, P], ctypes.c_int),
    "moe_topk": ([P, I64, I32, I32, ctypes.c_int, P, P, P], ctypes.c_int),
    "moe_permute_workspace_size": ([I64, I32, I32], SZ),
    "moe_permute": ([P, P, I64, I64, I32, I32, ctypes.c_int, P, P, P, P, P, P, SZ, P], ctypes.c_int),
    "moe_grouped_gemm_gateup_swiglu": ([P, P, P, I64, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_grouped_gemm_down": ([P, P, P, I64, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_unpermute_combine": ([P, P, P, P, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_decode_gateup_swiglu": ([P, P, P, I64, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_decode_down": ([P, P, P, I64, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_decode_gateup_swiglu_gather": ([P, P, I32, P, P, I64, I64, I64, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_grouped_gemm_gateup_swiglu_gather": ([P, P, I32, P, P, I64, I64, I64, I32, ctypes.c_int, P, P],
                                              ctypes.c_int),
    "moe_localize_ids": ([P, I64, I32, I32, P, P], ctypes.c_int),
    "moe_localize_ids_strided": ([P, I64, I32, I32, I32, P, P], ctypes.c_int),
    "moe_localize_ids_mapped": ([P, I64, P, I32, I32, P, P], ctypes.c_int),
    "moe_permute_noalloc": ([P, P, I64, I64, I32, I32, ctypes.c_int, P, P, P, P, P, P], ctypes.c_int),
    "moe_batched_gateup_swiglu": ([P, P, P, I64, I64, I64, I32, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_batched_down_combine": ([P, P, P, P, P, I64, I64, I64, I32, I32, ctypes.c_int, P, P], ctypes.c_int),
    "moe_decode_gateup_swiglu_mxfp4": ([P, P, I32, P, P, P, I64, I64, I64, I32, P, P], ctypes.c_int),
    "moe_decode_down_mxfp4": ([P, P, P, P, I64, I64, I64, I32, P, P], ctypes.c_int),
    "moe_batched_gateup_swiglu_mxfp4": ([P, P, P, P, I64, I64, I64, I32, I32, P, P], ctypes.c_int),
    "moe_batched_down_combine_mxfp4": ([P, P, P, P, P, P, I64, I64, I64, I32, I32, P, P], ctypes.c_int),
    "moe_batched_gateup_swiglu_select": ([P, P, P, I64, I64, I64, I32, I32, ctypes.c_int, ctypes.c_int, P, P, P, P],
                                         ctypes.c_int),
    "moe_batched_gateup_swiglu_mxfp4_select": ([P, P, P, P, I64, I64, I64, I32, I32, ctypes.c_int, P, P, P, P],
                                               ctypes.c_int),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = load().moe_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (after torch, so the HIP runtime torch loaded is the
    one the library binds to).  Raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libmoe.so not built ({path}); run __graft_entry__.build() "
                           "or python -m mixture_experts_ffn_04_amd.build")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


SCORES = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}


# ------------------------------------------------------------- single calls

def route(x, w_router, bias, k: int, score: str, logits, topk_ids, topk_w, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    _check("moe_route", load().moe_route(_ptr(x), _ptr(w_router), _ptr(bias), T, d, E, k, _dt(x),
                                         SCORES[score], _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                         _stream(stream)))


def topk(logits, k: int, score: str, topk_ids, topk_w, stream=None):
    T, E = logits.shape
    _check("moe_topk", load().moe_topk(_ptr(logits), T, E, k, SCORES[score], _ptr(topk_ids),
                                       _ptr(topk_w), _stream(stream)))


def localize_ids(topk_ids, e_begin: int, e_count: int, local_ids, e_stride: int = 1, stream=None):
    """Expert-parallel share: global ids -> ids local to the experts e_begin,
    e_begin + e_stride, ... (e_count of them), -1 elsewhere."""
    if e_stride == 1:
        _check("moe_localize_ids", load().moe_localize_ids(_ptr(topk_ids), topk_ids.numel(), e_begin, e_count,
                                                           _ptr(local_ids), _stream(stream)))
    else:
        _check("moe_localize_ids_strided", load().moe_localize_ids_strided(
            _ptr(topk_ids), topk_ids.numel(), e_begin, e_stride, e_count, _ptr(local_ids), _stream(stream)))


def localize_ids_mapped(topk_ids, expert_map, e_count: int, local_ids, stream=None):
    """Expert-parallel share holding any set of experts: global id e ->
    expert_map[e] (int32 [E] on the device, -1 for experts held elsewhere)."""
    _check("moe_localize_ids_mapped", load().moe_localize_ids_mapped(
        _ptr(topk_ids), topk_ids.numel(), _ptr(expert_map), expert_map.numel(), e_count, _ptr(local_ids),
        _stream(stream)))


def permute_workspace_size(T: int, k: int, E: int) -> int:
    return int(load().moe_permute_workspace_size(T, k, E))


def permute(topk_ids, x, E: int, counts, offsets, perm, inv_perm, x_perm, ws, stream=None):
    T, k = topk_ids.shape
    d = x.shape[1] if x is not None else 0
    dt = _dt(x) if x is not None else MOE_BF16
    _check("moe_permute", load().moe_permute(_ptr(topk_ids), _ptr(x), T, d, E, k, dt, _ptr(counts),
                                             _ptr(offsets), _ptr(perm), _ptr(inv_perm), _ptr(x_perm),
                                             _ptr(ws), ws.numel() * ws.element_size() if ws is not None else 0,
                                             _stream(stream)))


def permute_noalloc(topk_ids, x, E: int, counts, offsets, perm, inv_perm, x_perm, stream=None):
    """moe_permute with the library's own per-GPU scratch (no workspace)."""
    T, k = topk_ids.shape
    d = x.shape[1] if x is not None else 0
    dt = _dt(x) if x is not None else MOE_BF16
    _check("moe_permute_noalloc", load().moe_permute_noalloc(
        _ptr(topk_ids), _ptr(x), T, d, E, k, dt, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
        _ptr(x_perm), _stream(stream)))


def gateup_swiglu(x_perm, w_gate_up, offsets, h, decode: bool = False, stream=None):
    rows, d = x_perm.shape
    E, f2, _ = w_gate_up.shape
    fn = "moe_decode_gateup_swiglu" if decode else "moe_grouped_gemm_gateup_swiglu"
    _check(fn, getattr(load(), fn)(_ptr(x_perm), _ptr(w_gate_up), _ptr(offsets), rows, d, f2 // 2, E,
                                   _dt(x_perm), _ptr(h), _stream(stream)))


def gateup_swiglu_gather(x, perm, k: int, w_gate_up, offsets, h, decode: bool = False, stream=None):
    """Gate/up + SwiGLU reading row r as x[perm[r] // k] (no x_perm), grouped
    or decode form."""
    rows = perm.shape[0]
    d = x.shape[1]
    E, f2, _ = w_gate_up.shape
    fn = "moe_decode_gateup_swiglu_gather" if decode else "moe_grouped_gemm_gateup_swiglu_gather"
    _check(fn, getattr(load(), fn)(_ptr(x), _ptr(perm), k, _ptr(w_gate_up), _ptr(offsets), rows, d, f2 // 2, E,
                                   _dt(x), _ptr(h), _stream(stream)))


def down(h, w_down, offsets, y_perm, decode: bool = False, stream=None):
    rows, f = h.shape
    E, d, _ = w_down.shape
    fn = "moe_decode_down" if decode else "moe_grouped_gemm_down"
    _check(fn, getattr(load(), fn)(_ptr(h), _ptr(w_down), _ptr(offsets), rows, d, f, E, _dt(h),
                                   _ptr(y_perm), _stream(stream)))


def batched_gateup_swiglu(x, topk_ids, w_gate_up, h, stream=None):
    """The "batched_mm" gate/up: h [T*k, f] in pair order, no sort."""
    T, d = x.shape
    k = topk_ids.shape[1]
    E, f2, _ = w_gate_up.shape
    _check("moe_batched_gateup_swiglu", load().moe_batched_gateup_swiglu(
        _ptr(x), _ptr(topk_ids), _ptr(w_gate_up), T, d, f2 // 2, E, k, _dt(x), _ptr(h), _stream(stream)))


def batched_gateup_swiglu_select(x, logits, k: int, score: str, w_gate_up, topk_ids, topk_w, h, stream=None):
    """The "batched_mm" gate/up that selects each token's experts from the
    router logits itself (writing topk_ids / topk_w for the down call)."""
    T, d = x.shape
    E, f2, _ = w_gate_up.shape
    _check("moe_batched_gateup_swiglu_select", load().moe_batched_gateup_swiglu_select(
        _ptr(x), _ptr(logits), _ptr(w_gate_up), T, d, f2 // 2, E, k, SCORES[score], _dt(x), _ptr(topk_ids),
        _ptr(topk_w), _ptr(h), _stream(stream)))


def batched_gateup_swiglu_mxfp4_select(x, logits, k: int, score: str, wq_gate_up, ws_gate_up, topk_ids, topk_w, h,
                                       stream=None):
    """The same with MXFP4 expert weights."""
    T, d = x.shape
    E, f2, _ = wq_gate_up.shape
    _check("moe_batched_gateup_swiglu_mxfp4_select", load().moe_batched_gateup_swiglu_mxfp4_select(
        _ptr(x), _ptr(logits), _ptr(wq_gate_up), _ptr(ws_gate_up), T, d, f2 // 2, E, k, SCORES[score],
        _ptr(topk_ids), _ptr(topk_w), _ptr(h), _stream(stream)))


def batched_down_combine(h, topk_ids, topk_w, w_down, y_shared, y, stream=None):
    """The "batched_mm" down projection with the weighted combine folded in."""
    T, k = topk_ids.shape
    E, d, f = w_down.shape
    _check("moe_batched_down_combine", load().moe_batched_down_combine(
        _ptr(h), _ptr(topk_ids), _ptr(topk_w), _ptr(w_down), _ptr(y_shared), T, d, f, E, k, _dt(h), _ptr(y),
        _stream(stream)))


def gateup_swiglu_mxfp4(x, perm, k: int, wq_gate_up, ws_gate_up, offsets, h, stream=None):
    """Decode gate/up + SwiGLU with MXFP4 expert weights: row r is
    x[perm[r] // k], or x[r] when perm is None."""
    rows, f = h.shape
    E, _, dh = wq_gate_up.shape
    _check("moe_decode_gateup_swiglu_mxfp4", load().moe_decode_gateup_swiglu_mxfp4(
        _ptr(x), _ptr(perm), k, _ptr(wq_gate_up), _ptr(ws_gate_up), _ptr(offsets), rows, 2 * dh, f, E, _ptr(h),
        _stream(stream)))


def down_mxfp4(h, wq_down, ws_down, offsets, y_perm, stream=None):
    """Decode down projection with MXFP4 expert weights."""
    rows, f = h.shape
    E, d, _ = wq_down.shape
    _check("moe_decode_down_mxfp4", load().moe_decode_down_mxfp4(
        _ptr(h), _ptr(wq_down), _ptr(ws_down), _ptr(offsets), rows, d, f, E, _ptr(y_perm), _stream(stream)))


def batched_gateup_swiglu_mxfp4(x, topk_ids, wq_gate_up, ws_gate_up, h, stream=None):
    """The "batched_mm" gate/up with MXFP4 expert weights: h [T*k, f] in
    pair order, no sort."""
    T, d = x.shape
    k = topk_ids.shape[1]
    E, f2, _ = wq_gate_up.shape
    _check("moe_batched_gateup_swiglu_mxfp4", load().moe_batched_gateup_swiglu_mxfp4(
        _ptr(x), _ptr(topk_ids), _ptr(wq_gate_up), _ptr(ws_gate_up), T, d, f2 // 2, E, k, _ptr(h), _stream(stream)))


def batched_down_combine_mxfp4(h, topk_ids, topk_w, wq_down, ws_down, y_shared, y, stream=None):
    """The "batched_mm" down projection with MXFP4 expert weights and the
    weighted combine folded in."""
    T, k = topk_ids.shape
    E, d, fh = wq_down.shape
    _check("moe_batched_down_combine_mxfp4", load().moe_batched_down_combine_mxfp4(
        _ptr(h), _ptr(topk_ids), _ptr(topk_w), _ptr(wq_down), _ptr(ws_down), _ptr(y_shared), T, d, 2 * fh, E, k,
        _ptr(y), _stream(stream)))


def unpermute_combine(y_perm, inv_perm, topk_w, y_shared, y, stream=None):
    T, k = topk_w.shape
    d = y.shape[1]
    _check("moe_unpermute_combine", load().moe_unpermute_combine(
        _ptr(y_perm), _ptr(inv_perm), _ptr(topk_w), _ptr(y_shared), T, d, k, _dt(y), _ptr(y),
        _stream(stream)))


# ------------------------------------------------------------- whole layer

@dataclass
class MoeWeights:
    w_router: torch.Tensor           # [E, d]
    bias: Optional[torch.Tensor]     # [E] fp32 or None
    w_gate_up: torch.Tensor          # [E, 2f, d]
    w_down: torch.Tensor             # [E, d, f]
    shared_gate_up: Optional[torch.Tensor] = None   # [1, 2f_s, d]
    shared_down: Optional[torch.Tensor] = None      # [1, d, f_s]
    # MXFP4 experts: w_gate_up / w_down then hold uint8 codes ([E, 2f, d/2],
    # [E, d, f/2]) and these their E8M0 block scales ([E, 2f, d/32], [E, d, f/32])
    w_gate_up_scales: Optional[torch.Tensor] = None
    w_down_scales: Optional[torch.Tensor] = None

    @property
    def mxfp4(self) -> bool:
        return self.w_gate_up_scales is not None


class MoeLayer:
    """The routed MoE FFN layer over preallocated device buffers.

    forward(x) enqueues, on the current stream: moe_route, moe_permute,
    gate/up + SwiGLU and down projections (grouped, or decode variants for
    small batches), the shared expert when present, and the weighted
    combine.  Buffers are allocated once per token count and reused.

    mode: "grouped" (sort by expert, grouped GEMMs), "decode" (sort, then
    the decode calls that stream only the active experts' weights),
    "batched" (the small-batch "batched_mm" strategy: per (token, slot)
    pair, no sort, the combine folded into the down call) or "auto"
    ("batched" for one bf16 token, decode up to DECODE_MAX_ROWS routed
    rows, grouped above).

    experts=(e_begin, e_count) makes it one expert-parallel share: the
    router (weights.w_router) covers all experts, weights.w_gate_up and
    weights.w_down hold only experts [e_begin, e_begin + e_count) (with
    experts=(e_begin, e_count, e_stride) the experts e_begin, e_begin +
    e_stride, ..., in that order: an interleaved assignment), and
    forward returns the share's partial output (the pairs of other experts
    masked by moe_localize_ids); the partial outputs of all shares sum to
    the layer's output.  expert_ids=[e0, e1, ...] instead names any set of
    global experts that the weights hold, in that order (moe_localize_ids_mapped;
    see placement.balanced_shares).

    shared_part=(i, n) runs the shared expert (when the weights hold it)
    on tokens [T i / n, T (i + 1) / n) only, so that n shares that each
    hold it split its work: the partial output has the shared expert's
    rows of that slice and zeros for it elsewhere.
    """

    DECODE_MAX_ROWS = 256

    def __init__(self, weights: MoeWeights, k: int, score: str, mode: str = "auto",
                 experts: Optional[tuple] = None, overlap_shared: bool = False,
                 shared_part: Optional[tuple] = None, expert_ids=None):
        load()
        self.w = weights
        # the shared expert does not depend on the routing: with
        # overlap_shared (grouped calls) it runs on a second stream from the
        # start of the layer, beside the router, the sort and the routed
        # projections, and the combine waits for it
        self.overlap_shared = overlap_shared
        self._side = None
        self.k = k
        self.score = score
        self.mode = mode
        self.E, self.d = weights.w_router.shape          # experts seen by the router
        self.E_loc = weights.w_gate_up.shape[0]          # experts held here
        self.emap = None
        if experts is not None and expert_ids is not None:
            raise ValueError("pass experts=(e_begin, e_count[, e_stride]) or expert_ids, not both")
        if expert_ids is not None:
            held = [int(e) for e in expert_ids]
            if len(held) != self.E_loc:
                raise ValueError("expert_ids must name as many experts as the weights hold")
            self.emap = torch.tensor(expert_map(held, self.E), dtype=torch.int32, device=weights.w_router.device)
            self.e_begin = 0                             # a share: ids are localised
            self.e_stride = 1
        elif experts is None:
            if self.E_loc != self.E:
                raise ValueError("expert weights cover a share of the experts: pass experts=(e_begin, e_count)")
            self.e_begin = None
        else:
            e_begin, e_count = experts[:2]
            e_stride = experts[2] if len(experts) > 2 else 1
            if (e_count != self.E_loc or e_begin < 0 or e_stride < 1
                    or e_begin + (e_count - 1) * e_stride >= self.E):
                raise ValueError("experts=(e_begin, e_count[, e_stride]) does not match the expert weights")
            self.e_begin = int(e_begin)
            self.e_stride = int(e_stride)
        if shared_part is not None:
            i, n = shared_part
            if n < 1 or not 0 <= i < n:
                raise ValueError("shared_part=(i, n) needs 0 <= i < n")
        self.shared_part = shared_part
        self.mx = weights.mxfp4
        self.f = weights.w_down.shape[2] * (2 if self.mx else 1)
        self.dev = weights.w_router.device
        self.dtype = weights.w_router.dtype             # activations
        if self.mx and mode not in ("auto", "decode", "batched"):
            raise ValueError("MXFP4 experts run on the decode or the batched calls")
        self._T = None

    def _alloc(self, T: int):
        if self._T == T:
            return
        if self._side is not None:
            # buffers the second stream may still use are about to be freed
            torch.cuda.current_stream(self.dev).wait_stream(self._side)
        dev, dt, k, E, d, f = self.dev, self.dtype, self.k, self.E, self.d, self.f
        P = T * k
        i32 = torch.int32
        self.logits = torch.empty(T, E, device=dev, dtype=torch.float32)
        self.ids = torch.empty(T, k, device=dev, dtype=i32)
        self.wts = torch.empty(T, k, device=dev, dtype=torch.float32)
        El = self.E_loc
        self.counts = torch.empty(El, device=dev, dtype=i32)
        self.offsets = torch.empty(El + 1, device=dev, dtype=i32)
        self.lids = torch.empty(T, k, device=dev, dtype=i32) if self.e_begin is not None else None
        self.perm = torch.empty(P, device=dev, dtype=i32)
        self.inv_perm = torch.empty(P, device=dev, dtype=i32)
        self.x_perm = torch.empty(P, d, device=dev, dtype=dt)
        self.h = torch.empty(P, f, device=dev, dtype=dt)
        self.y_perm = torch.empty(P, d, device=dev, dtype=dt)
        self.ws = torch.empty(max(1, permute_workspace_size(T, k, El)), device=dev, dtype=torch.uint8)
        self.y = torch.empty(T, d, device=dev, dtype=dt)
        if self.w.shared_gate_up is not None:
            fs = self.w.shared_down.shape[2]
            t0, t1 = self.shared_rows(T)
            self.s_off = torch.tensor([0, t1 - t0], device=dev, dtype=i32)
            self.s_h = torch.empty(t1 - t0, fs, device=dev, dtype=dt)
            # rows outside the slice are never written: zero once
            self.s_y = (torch.zeros if (t0, t1) != (0, T) else torch.empty)(T, d, device=dev, dtype=dt)
        self._T = T

    def _localize_stage(self, st) -> tuple:
        if self.emap is not None:
            return ("localize", localize_ids_mapped, (self.ids, self.emap, self.E_loc, self.lids, st))
        return ("localize", localize_ids, (self.ids, self.e_begin, self.E_loc, self.lids, self.e_stride, st))

    def shared_rows(self, T: int) -> tuple:
        """The tokens [t0, t1) this layer runs the shared expert on."""
        if self.shared_part is None:
            return 0, T
        i, n = self.shared_part
        return T * i // n, T * (i + 1) // n

    def use_batched(self, T: int) -> bool:
        """The "batched_mm" strategy: when asked for, and in "auto" for a
        single token with bf16 activations, bf16 or MXFP4 experts (its k
        experts are distinct, so each expert's weights are read once either
        way, and the sort and the combine launches are saved)."""
        if self.mode == "batched":
            return True
        return self.mode == "auto" and T == 1 and self.dtype == torch.bfloat16

    def use_decode(self, T: int) -> bool:
        if self.mode == "decode":
            return True
        if self.mode in ("grouped", "batched"):
            return False
        return T * self.k <= self.DECODE_MAX_ROWS

    STAGES = ("route", "localize", "permute", "gateup", "down", "shared_gateup", "shared_down", "combine")

    def stages(self, x: torch.Tensor, st) -> list:
        """The layer on x [T, d] as (stage name, call, args) in launch order."""
        T = x.shape[0]
        self._alloc(T)
        w = self.w
        if self.use_batched(T):
            return self._batched_stages(x, st)
        dec = self.use_decode(T)
        if self.mx and T * self.k > 1024:
            raise ValueError("MXFP4 experts: at most 1024 routed rows (the decode calls)")
        # bf16 gate/up reads the token rows through the sort (no x_perm copy)
        gather = self.dtype == torch.bfloat16
        out = [("route", route, (x, w.w_router, w.bias, self.k, self.score, self.logits, self.ids, self.wts, st))]
        ids = self.ids
        if self.e_begin is not None:
            out.append(self._localize_stage(st))
            ids = self.lids
        out += [
            ("permute", permute, (ids, x, self.E_loc, self.counts, self.offsets, self.perm, self.inv_perm,
                                  None if gather else self.x_perm, self.ws, st)),
            ("gateup", gateup_swiglu_gather, (x, self.perm, self.k, w.w_gate_up, self.offsets, self.h, dec, st))
            if gather else
            ("gateup", gateup_swiglu, (self.x_perm, w.w_gate_up, self.offsets, self.h, dec, st)),
            ("down", down, (self.h, w.w_down, self.offsets, self.y_perm, dec, st)),
        ]
        if self.mx:
            out[-2:] = [
                ("gateup", gateup_swiglu_mxfp4, (x, self.perm, self.k, w.w_gate_up, w.w_gate_up_scales, self.offsets,
                                                 self.h, st)),
                ("down", down_mxfp4, (self.h, w.w_down, w.w_down_scales, self.offsets, self.y_perm, st)),
            ]
        ys = None
        if w.shared_gate_up is not None:
            t0, t1 = self.shared_rows(T)
            sdec = dec and t1 - t0 <= self.DECODE_MAX_ROWS
            ss = st
            if self.overlap_shared and not sdec:
                if self._side is None:
                    self._side = torch.cuda.Stream(device=self.dev)     # default priority
                ss = self._side
            sh = [("shared_gateup", gateup_swiglu, (x[t0:t1], w.shared_gate_up, self.s_off, self.s_h, sdec, ss)),
                  ("shared_down", down, (self.s_h, w.shared_down, self.s_off, self.s_y[t0:t1], sdec, ss))]
            sh = sh if t1 > t0 else []
            ys = self.s_y
            out = sh + out if ss is not st else out + sh
        out.append(("combine", unpermute_combine, (self.y_perm, self.inv_perm, self.wts, ys, self.y, st)))
        return out

    def _batched_stages(self, x: torch.Tensor, st) -> list:
        """The "batched_mm" strategy: the router logits, then per (token,
        slot) pair the gate/up projection, which also selects the experts
        from the logits (the router's top-k launch saved), and the down
        projection with the weighted combine folded in; no sort.  On an
        expert-parallel share the router selects and the ids are localised
        first.  The shared expert runs on the decode calls before the down
        projection, which adds its output."""
        T = x.shape[0]
        w = self.w
        if self.mx and T * self.k > 1024:
            raise ValueError("MXFP4 experts: at most 1024 routed rows (the batched calls)")
        select = self.e_begin is None
        ids = self.ids
        if select:
            out = [("route", route, (x, w.w_router, w.bias, self.k, self.score, self.logits, None, None, st))]
        else:
            out = [("route", route, (x, w.w_router, w.bias, self.k, self.score, self.logits, self.ids, self.wts, st)),
                   self._localize_stage(st)]
            ids = self.lids
        ys = None
        if w.shared_gate_up is not None:
            t0, t1 = self.shared_rows(T)
            if t1 > t0:
                out.append(("shared_gateup", gateup_swiglu,
                            (x[t0:t1], w.shared_gate_up, self.s_off, self.s_h, True, st)))
                out.append(("shared_down", down, (self.s_h, w.shared_down, self.s_off, self.s_y[t0:t1], True, st)))
            ys = self.s_y
        if self.mx:
            if select:
                out.append(("gateup", batched_gateup_swiglu_mxfp4_select,
                            (x, self.logits, self.k, self.score, w.w_gate_up, w.w_gate_up_scales, self.ids, self.wts,
                             self.h, st)))
            else:
                out.append(("gateup", batched_gateup_swiglu_mxfp4,
                            (x, ids, w.w_gate_up, w.w_gate_up_scales, self.h, st)))
            out.append(("down", batched_down_combine_mxfp4, (self.h, ids, self.wts, w.w_down, w.w_down_scales, ys,
                                                             self.y, st)))
        else:
            if select:
                out.append(("gateup", batched_gateup_swiglu_select,
                            (x, self.logits, self.k, self.score, w.w_gate_up, self.ids, self.wts, self.h, st)))
            else:
                out.append(("gateup", batched_gateup_swiglu, (x, ids, w.w_gate_up, self.h, st)))
            out.append(("down", batched_down_combine, (self.h, ids, self.wts, w.w_down, ys, self.y, st)))
        return out

    def forward(self, x: torch.Tensor, stream=None, marks: Optional[dict] = None,
                stages: Optional[tuple] = None, run: Optional[tuple] = None) -> torch.Tensor:
        """Run the layer on x [T, d].  With `marks` (a dict), a pair of timing
        events recorded on the launch stream brackets every stage (or only the
        stages named in `stages`) and is appended to marks[stage].  With
        `run`, only the stages named there are enqueued."""
        st = torch.cuda.current_stream() if stream is None else stream
        side = None
        for name, fn, a in self.stages(x, st):
            if run is not None and name not in run:
                continue
            s = a[-1]                                # the stage's launch stream
            if s is not st and side is None:
                side = s
                side.wait_stream(st)                 # x and the buffers are ready
            if name == "combine" and side is not None:
                st.wait_stream(side)                 # the shared expert's output is ready
            if marks is None or (stages is not None and name not in stages):
                fn(*a)
                continue
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            fn(*a)
            e1.record(s)
            marks.setdefault(name, []).append((e0, e1))
        return self.y


class MoeLayerGraph:
    """One forward of the layer at a fixed token count T, captured in HIP
    graphs: a replay costs one graph launch per segment instead of one host
    call per stage, which is what bounds a decode step.

    The graphs own their buffers (a private MoeLayer over the same weights)
    and a static input `x` [T, d]: write the tokens into `x`, then call
    replay(), which enqueues the layer on the current stream and returns the
    static output [T, d].  Each stage named in `timed` is captured as a
    segment of its own and bracketed by timing events on the stream between
    segment replays; stage_ms() reads them for the last replay once it has
    completed.  Replays of one MoeLayerGraph must not overlap.
    """

    def __init__(self, weights: MoeWeights, k: int, score: str, T: int, mode: str = "auto",
                 timed: tuple = ()):
        self.layer = L = MoeLayer(weights, k, score, mode)
        self.T = T
        self.x = torch.zeros(T, L.d, dtype=L.dtype, device=L.dev)
        side = torch.cuda.Stream(device=L.dev)
        side.wait_stream(torch.cuda.current_stream(L.dev))
        with torch.cuda.stream(side):
            L.forward(self.x)                    # allocates the buffers outside the capture
        torch.cuda.current_stream(L.dev).wait_stream(side)
        torch.cuda.synchronize(L.dev)
        names = [n for n, _, _ in L.stages(self.x, side)]
        segs, cur = [], []
        for n in names:
            if n in timed:
                if cur:
                    segs.append((tuple(cur), False))
                segs.append(((n,), True))
                cur = []
            else:
                cur.append(n)
        if cur:
            segs.append((tuple(cur), False))
        self.segments = []
        for run, is_timed in segs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                L.forward(self.x, run=run)
            self.segments.append((run, is_timed, g))
        self.y = L.y
        self._ev = {}

    def replay(self) -> torch.Tensor:
        st = torch.cuda.current_stream(self.layer.dev)
        for run, is_timed, g in self.segments:
            if is_timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                g.replay()
                e1.record(st)
                self._ev[run[0]] = (e0, e1)
            else:
                g.replay()
        return self.y

    def stage_ms(self) -> dict:
        return {name: e0.elapsed_time(e1) for name, (e0, e1) in self._ev.items()}


# The C ABI's own names, for callers that mirror include/libmoe.h.
moe_route = route
moe_topk = topk
moe_permute_workspace_size = permute_workspace_size
moe_permute = permute
moe_permute_noalloc = permute_noalloc
moe_grouped_gemm_gateup_swiglu = gateup_swiglu
moe_grouped_gemm_down = down
moe_unpermute_combine = unpermute_combine
moe_localize_ids = localize_ids


def moe_decode_gateup_swiglu(x_perm, w_gate_up, offsets, h, stream=None):
    gateup_swiglu(x_perm, w_gate_up, offsets, h, True, stream)


def moe_decode_down(h, w_down, offsets, y_perm, stream=None):
    down(h, w_down, offsets, y_perm, True, stream)


def moe_decode_gateup_swiglu_gather(x, perm, k, w_gate_up, offsets, h, stream=None):
    gateup_swiglu_gather(x, perm, k, w_gate_up, offsets, h, True, stream)


def moe_grouped_gemm_gateup_swiglu_gather(x, perm, k, w_gate_up, offsets, h, stream=None):
    gateup_swiglu_gather(x, perm, k, w_gate_up, offsets, h, False, stream)
