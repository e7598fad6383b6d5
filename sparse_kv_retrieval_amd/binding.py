"""ctypes binding of libdualkv for torch tensors and torch streams.

Argument marshalling only: each function checks that tensors have the layout
the C ABI states, passes their data pointers and the current HIP stream, and
raises ``DualKVError`` when the library returns anything but DK_OK.  Every step
of the computation runs in the library's HIP kernels; torch provides memory and
streams.  Importing this module fails loudly if ``libdualkv.so`` has not been
built (``python -m sparse_kv_retrieval_amd.build``).
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdualkv.so")

DK_OK, DK_ERR_INVALID_ARG, DK_ERR_UNSUPPORTED, DK_ERR_HIP = 0, 1, 2, 3
DK_F32, DK_BF16 = 0, 1
DK_REDUCE_MEAN, DK_REDUCE_MAX = 0, 1
ABI_VERSION = 14

_STATUS = {0: "DK_OK", 1: "DK_ERR_INVALID_ARG", 2: "DK_ERR_UNSUPPORTED", 3: "DK_ERR_HIP"}


class DualKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class dk_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("t", ctypes.c_int64)]


class dk_landmark_shadow(ctypes.Structure):
    _fields_ = [("lm8", ctypes.c_void_p), ("chunk_scale", ctypes.c_void_p), ("scale_max", ctypes.c_void_p)]


class dk_cache_plan(ctypes.Structure):
    _fields_ = [("resident", ctypes.c_void_p), ("slots", ctypes.c_int),
                ("slot_of_union", ctypes.c_void_p), ("miss_chunk", ctypes.c_void_p),
                ("miss_slot", ctypes.c_void_p), ("miss_count", ctypes.c_void_p),
                ("hit_count", ctypes.c_void_p)]


class dk_attn_extra(ctypes.Structure):
    _fields_ = [("K_tail", ctypes.c_void_p), ("V_tail", ctypes.c_void_p), ("tail_k_s", dk_strides),
                ("tail_v_s", dk_strides), ("tail_len", ctypes.c_void_p), ("tail_max", ctypes.c_int),
                ("K_new", ctypes.c_void_p), ("V_new", ctypes.c_void_p)]


# (name, restype, argtypes) of every exported function
_P, _I, _Z, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float, dk_strides
EXPORTS = [
    ("dk_abi_version", ctypes.c_int, []),
    ("dk_last_error", ctypes.c_char_p, []),
    ("dk_build_landmarks", _I, [_P, _I, _S, _I, _I, _I, _I, _I, _P, _P]),
    ("dk_build_landmark_shadow", _I, [_P, _S, _I, _I, _I, _I, _P, _P, _P, _P]),
    ("dk_score_topk_workspace_size", _Z, [_I, _I, _I, _I, _I, _I]),
    ("dk_index_topk_workspace_size", _Z, [_I, _I, _I, _I]),
    ("dk_build_minmax", _I, [_P, _I, _S, _I, _I, _I, _I, _I, _P, _P, _P]),
    ("dk_score_topk_minmax", _I, [_P, _I, _I, _I, _P, _P, _I, _S, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _P, _P,
                                  _P, _Z, _P]),
    ("dk_coverage_workspace_size", _Z, [_I, _I, _I, _I]),
    ("dk_score_coverage", _I, [_P, _I, _I, _I, _P, _I, _S, _I, _I, _I, _F, _I, _F, _I, _P, _P, _P, _P, _P, _P, _P,
                               _P, _Z, _P]),
    ("dk_score_topk", _I, [_P, _I, _I, _I, _P, _I, _S, _I, _I, _I, _I, _F, _I,
                           ctypes.POINTER(dk_landmark_shadow), _P, _P, _P, _Z, _P]),
    ("dk_score_topk_union", _I, [_P, _I, _I, _I, _P, _I, _S, _I, _I, _I, _I, _F, _I,
                                 ctypes.POINTER(dk_landmark_shadow), _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    ("dk_decode_step_workspace_size", _Z, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    ("dk_decode_step", _I, [_P, _I, _I, _I, _I, _P, _I, _S, _I, _I, _I, _F, _I, ctypes.POINTER(dk_landmark_shadow),
                            _P, _P, _I, _S, _S, _I, ctypes.POINTER(dk_attn_extra), _P, _P, _P, _P, _P, _P, _P, _P,
                            _P, _Z, _P]),
    ("dk_capped_plan", _I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    ("dk_union_select", _I, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, ctypes.POINTER(dk_cache_plan), _P]),
    ("dk_gather_kv", _I, [_P, _P, _I, _S, _I, _I, _I, _I, _P, _P, _P, _I, _I, _P, _P, _S, _I, _I, _P]),
    ("dk_attn_workspace_size", _Z, [_I, _I, _I, _I, _I, _I, _I]),
    ("dk_sparse_decode_attn", _I, [_P, _I, _I, _I, _I, _P, _P, _I, _S, _S, _I, _I, _I, _P, _P, _P,
                                   _I, _I, _F, _P, _P, _P, _Z, _P]),
    ("dk_sparse_decode_attn_noalloc", _I, [_P, _I, _I, _I, _I, _P, _P, _I, _S, _S, _I, _I, _I, _P, _P, _P,
                                           _I, _I, _F, _P, _P, _P]),
    ("dk_attn_tail_workspace_size", _Z, [_I, _I, _I, _I, _I, _I, _I]),
    ("dk_sparse_decode_attn_tail", _I, [_P, _I, _I, _I, _I, _P, _P, _I, _S, _S, _I, _I, _I, _P, _P, _P,
                                        _I, _I, ctypes.POINTER(dk_attn_extra), _F, _P, _P, _P, _Z, _P]),
]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdualkv.so not found at {LIB_PATH}; build it with "
                          "`python -m sparse_kv_retrieval_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in EXPORTS:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.dk_abi_version() != ABI_VERSION:
        raise ImportError(f"libdualkv ABI {lib.dk_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


lib = _load()


def _check(status: int):
    if status != DK_OK:
        raise DualKVError(status, lib.dk_last_error().decode(errors="replace"))


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_stream(fn):
    """Run a wrapper with its `stream` argument (when given) as torch's current
    stream, so that every buffer the wrapper allocates (outputs, workspaces)
    belongs to the stream its library call is enqueued on: the caching allocator
    then never hands that memory out again while the call may still use it."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, **kw)
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(s):
            return fn(*args, stream=s, **kw)
    return run


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DK_BF16
    if t.dtype == torch.float32:
        return DK_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def pool_strides(t: torch.Tensor) -> dk_strides:
    """dk_strides of a [B, H, rows, d] tensor whose last dimension is dense."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("pool tensors must be 4-D [B, H, rows, d] with a dense last dimension")
    s = t.stride()
    return dk_strides(s[0], s[1], s[2])


def _need(t: torch.Tensor, dtype, shape, name, device=True):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: need contiguous {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if device and not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


# ----------------------------------------------------------------------------
# one wrapper per C entry point
# ----------------------------------------------------------------------------

@_on_stream
def build_landmarks(K: torch.Tensor, chunk: int, lm: torch.Tensor | None = None, stream=None):
    B, H, L, d = K.shape
    C = L // chunk if chunk > 0 else 0
    if lm is None:
        lm = torch.empty(B, H, C, d, dtype=torch.float32, device=K.device)
    _need(lm, torch.float32, (B, H, C, d), "lm")
    _check(lib.dk_build_landmarks(_ptr(K), _dtype(K), pool_strides(K), B, H, L, d, chunk,
                                  _ptr(lm), _stream(stream)))
    return lm


@dataclass
class Shadow:
    """8-bit landmark codes, per-chunk scales and the per-(b, g) largest scale (dk_landmark_shadow)."""
    lm8: torch.Tensor          # [B, Hkv, C, d] uint8: rint(lm / scale) + 128
    chunk_scale: torch.Tensor  # [B, Hkv, C] float32: max |lm| / 127 per chunk
    scale_max: torch.Tensor    # [B, Hkv] float32: largest chunk scale, +inf if a landmark is not finite

    def as_c(self) -> dk_landmark_shadow:
        return dk_landmark_shadow(self.lm8.data_ptr(), self.chunk_scale.data_ptr(), self.scale_max.data_ptr())


@_on_stream
def build_landmark_shadow(lm: torch.Tensor, stream=None) -> Shadow:
    B, H, C, d = lm.shape
    dev = lm.device
    sh = Shadow(torch.empty(B, H, C, d, dtype=torch.uint8, device=dev),
                torch.empty(B, H, C, dtype=torch.float32, device=dev),
                torch.empty(B, H, dtype=torch.float32, device=dev))
    _check(lib.dk_build_landmark_shadow(_ptr(lm), pool_strides(lm), B, H, C, d, _ptr(sh.lm8), _ptr(sh.chunk_scale),
                                        _ptr(sh.scale_max), _stream(stream)))
    return sh


def score_topk_workspace_size(B, Hkv, T, C, k, with_shadow=False) -> int:
    return int(lib.dk_score_topk_workspace_size(B, Hkv, T, C, k, int(bool(with_shadow))))


def index_topk_workspace_size(B, Hkv, T, C) -> int:
    """Workspace of score_topk / score_topk_union with bf16 per-token indexer keys."""
    return int(lib.dk_index_topk_workspace_size(B, Hkv, T, C))


def _topk_ws_bytes(lm, B, Hkv, T, C, k, shadow) -> int:
    if lm.dtype == torch.bfloat16:
        return index_topk_workspace_size(B, Hkv, T, C)
    return score_topk_workspace_size(B, Hkv, T, C, k, shadow is not None)


@_on_stream
def score_topk(q: torch.Tensor, lm: torch.Tensor, k: int, scale: float, reduce: int = DK_REDUCE_MEAN,
               topk_idx=None, topk_score=None, ws=None, want_scores=True, shadow: Shadow | None = None,
               stream=None):
    B, T, Hq, d = q.shape
    _, Hkv, C, _ = lm.shape
    _need(q, torch.float32, (B, T, Hq, d), "q")
    if topk_idx is None:
        topk_idx = torch.empty(B, Hkv, T, k, dtype=torch.int32, device=q.device)
    if topk_score is None and want_scores:
        topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=q.device)
    nbytes = _topk_ws_bytes(lm, B, Hkv, T, C, k, shadow)
    if ws is None and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    csh = ctypes.byref(shadow.as_c()) if shadow is not None else None
    _check(lib.dk_score_topk(_ptr(q), B, T, Hq, _ptr(lm), _dtype(lm), pool_strides(lm), Hkv, C, d, k,
                             float(scale), int(reduce), csh, _ptr(topk_idx), _ptr(topk_score),
                             _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                             _stream(stream)))
    return topk_idx, topk_score


@_on_stream
def build_minmax(K: torch.Tensor, chunk: int, kmin=None, kmax=None, stream=None):
    """Coordinate-wise min and max key of every chunk, [B, Hkv, L/chunk, d] in K's dtype."""
    B, Hkv, L, d = K.shape
    C = L // chunk
    if kmin is None:
        kmin = torch.empty(B, Hkv, C, d, dtype=K.dtype, device=K.device)
    if kmax is None:
        kmax = torch.empty(B, Hkv, C, d, dtype=K.dtype, device=K.device)
    _check(lib.dk_build_minmax(_ptr(K), _dtype(K), pool_strides(K), B, Hkv, L, d, chunk, _ptr(kmin), _ptr(kmax),
                               _stream(stream)))
    return kmin, kmax


@_on_stream
def score_topk_minmax(q: torch.Tensor, kmin: torch.Tensor, kmax: torch.Tensor, k: int, scale: float,
                      reduce: int = DK_REDUCE_MEAN, topk_idx=None, topk_score=None, union=False, union_ids=None,
                      member=None, count=None, overlap=None, ws=None, want_scores=True, stream=None):
    """Top-k chunks by min/max upper-bound scores; with union=True also the union outputs."""
    B, T, Hq, d = q.shape
    _, Hkv, C, _ = kmin.shape
    _need(q, torch.float32, (B, T, Hq, d), "q")
    if kmin.stride() != kmax.stride() or kmin.dtype != kmax.dtype:
        raise ValueError("kmin and kmax must share dtype and layout")
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty(B, Hkv, T, k, **i32)
    if topk_score is None and want_scores:
        topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=dev)
    if union:
        union_ids = torch.empty(B, Hkv, T * k, **i32) if union_ids is None else union_ids
        member = torch.empty(B, Hkv, T * k, dtype=torch.uint8, device=dev) if member is None else member
        count = torch.empty(B, Hkv, **i32) if count is None else count
        overlap = torch.empty(B, Hkv, **i32) if overlap is None else overlap
    nbytes = index_topk_workspace_size(B, Hkv, T, C)
    if ws is None:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib.dk_score_topk_minmax(_ptr(q), B, T, Hq, _ptr(kmin), _ptr(kmax), _dtype(kmin), pool_strides(kmin),
                                    Hkv, C, d, k, float(scale), int(reduce), _ptr(topk_idx), _ptr(topk_score),
                                    _ptr(union_ids), _ptr(member), _ptr(count), _ptr(overlap), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))
    if union:
        return topk_idx, topk_score, union_ids, member, count, overlap
    return topk_idx, topk_score


def coverage_workspace_size(B, Hkv, T, C) -> int:
    return int(lib.dk_coverage_workspace_size(B, Hkv, T, C))


@_on_stream
def score_coverage(q: torch.Tensor, lm: torch.Tensor, gamma: float, k_max: int, scale: float,
                   reduce: int = DK_REDUCE_MEAN, sel_idx=None, sel_count=None, sel_score=None, union=False,
                   union_ids=None, member=None, count=None, overlap=None, ws=None, want_scores=True, stream=None):
    """Smallest chunk sets reaching a fraction gamma of the softmax mass of the chunk scores.

    Returns (sel_idx [B, Hkv, T, k_max] ascending then -1, sel_count [B, Hkv, T], sel_score or None),
    followed by the union outputs (T * k_max slots) when union=True.
    """
    B, T, Hq, d = q.shape
    _, Hkv, C, _ = lm.shape
    _need(q, torch.float32, (B, T, Hq, d), "q")
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    if sel_idx is None:
        sel_idx = torch.empty(B, Hkv, T, k_max, **i32)
    if sel_count is None:
        sel_count = torch.empty(B, Hkv, T, **i32)
    if sel_score is None and want_scores:
        sel_score = torch.empty(B, Hkv, T, k_max, dtype=torch.float32, device=dev)
    if union:
        union_ids = torch.empty(B, Hkv, T * k_max, **i32) if union_ids is None else union_ids
        member = torch.empty(B, Hkv, T * k_max, dtype=torch.uint8, device=dev) if member is None else member
        count = torch.empty(B, Hkv, **i32) if count is None else count
        overlap = torch.empty(B, Hkv, **i32) if overlap is None else overlap
    if ws is None:
        ws = torch.empty(max(coverage_workspace_size(B, Hkv, T, C), 1), dtype=torch.uint8, device=dev)
    _check(lib.dk_score_coverage(_ptr(q), B, T, Hq, _ptr(lm), _dtype(lm), pool_strides(lm), Hkv, C, d, float(scale),
                                 int(reduce), float(gamma), int(k_max), _ptr(sel_idx), _ptr(sel_count),
                                 _ptr(sel_score), _ptr(union_ids), _ptr(member), _ptr(count), _ptr(overlap),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    if union:
        return sel_idx, sel_count, sel_score, union_ids, member, count, overlap
    return sel_idx, sel_count, sel_score


@_on_stream
def capped_plan(sel_ids: torch.Tensor, resident: torch.Tensor, stamp: torch.Tensor, cap: int, step: int,
                sel_score: torch.Tensor | None = None, sel_count: torch.Tensor | None = None, sel_slot=None,
                admit_chunk=None, admit_slot=None, admit_count=None, hit_count=None, stream=None):
    """One step of capped eviction: updates resident/stamp [B, Hkv, S] in place.

    sel_ids: [B, Hkv, N] (or a strided view of one query's rows, e.g. topk_idx[:, :, t]) with ascending ids;
    sel_score: the same layout or None; sel_count: [B, Hkv] (or a view with one stride) or None.
    Returns (sel_slot [B, Hkv, N], admit_chunk [B, Hkv, cap], admit_slot, admit_count [B, Hkv], hit_count).
    """
    B, Hkv, N = sel_ids.shape
    S = resident.shape[2]
    for name, t in (("resident", resident), ("stamp", stamp)):
        _need(t, torch.int32, (B, Hkv, S), name)
    if sel_ids.dtype != torch.int32 or sel_ids.stride(2) != 1 or sel_ids.stride(0) != Hkv * sel_ids.stride(1):
        raise ValueError("sel_ids must be int32 rows of unit stride, (b, g) rows at one stride")
    stride = sel_ids.stride(1)
    if sel_score is not None and (sel_score.dtype != torch.float32 or sel_score.shape != sel_ids.shape
                                  or sel_score.stride() != sel_ids.stride()):
        raise ValueError("sel_score must be float32 in the layout of sel_ids")
    cstride = 1
    if sel_count is not None:
        if sel_count.dtype != torch.int32 or sel_count.shape != (B, Hkv) or sel_count.stride(0) != Hkv * sel_count.stride(1):
            raise ValueError("sel_count must be int32 [B, Hkv] with one stride")
        cstride = sel_count.stride(1)
    dev = sel_ids.device
    i32 = dict(dtype=torch.int32, device=dev)
    sel_slot = torch.empty(B, Hkv, N, **i32) if sel_slot is None else sel_slot
    admit_chunk = torch.empty(B, Hkv, max(cap, 1), **i32) if admit_chunk is None else admit_chunk
    admit_slot = torch.empty(B, Hkv, max(cap, 1), **i32) if admit_slot is None else admit_slot
    admit_count = torch.empty(B, Hkv, **i32) if admit_count is None else admit_count
    hit_count = torch.empty(B, Hkv, **i32) if hit_count is None else hit_count
    _check(lib.dk_capped_plan(_ptr(sel_ids), _ptr(sel_score), _ptr(sel_count), B, Hkv, N, stride, cstride,
                              _ptr(resident), _ptr(stamp), S, int(cap), int(step), _ptr(sel_slot), _ptr(admit_chunk),
                              _ptr(admit_slot), _ptr(admit_count), _ptr(hit_count), _stream(stream)))
    return sel_slot, admit_chunk[..., :cap], admit_slot[..., :cap], admit_count, hit_count


@_on_stream
def score_topk_union(q: torch.Tensor, lm: torch.Tensor, k: int, scale: float,
                     reduce: int = DK_REDUCE_MEAN, topk_idx=None, topk_score=None, union_ids=None,
                     member=None, count=None, overlap=None, ws=None, want_scores=False,
                     shadow: Shadow | None = None, stream=None):
    """score_topk followed by union_select (no cache plan), as one library call."""
    B, T, Hq, d = q.shape
    _, Hkv, C, _ = lm.shape
    _need(q, torch.float32, (B, T, Hq, d), "q")
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty(B, Hkv, T, k, **i32)
    if topk_score is None and want_scores:
        topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=dev)
    if union_ids is None:
        union_ids = torch.empty(B, Hkv, T * k, **i32)
    if member is None:
        member = torch.empty(B, Hkv, T * k, dtype=torch.uint8, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, **i32)
    if overlap is None:
        overlap = torch.empty(B, Hkv, **i32)
    nbytes = _topk_ws_bytes(lm, B, Hkv, T, C, k, shadow)
    if ws is None and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    csh = ctypes.byref(shadow.as_c()) if shadow is not None else None
    _check(lib.dk_score_topk_union(_ptr(q), B, T, Hq, _ptr(lm), _dtype(lm), pool_strides(lm), Hkv, C, d,
                                   k, float(scale), int(reduce), csh, _ptr(topk_idx), _ptr(topk_score),
                                   _ptr(union_ids), _ptr(member), _ptr(count), _ptr(overlap), _ptr(ws),
                                   0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_score, union_ids, member, count, overlap


@dataclass
class CachePlan:
    """Device buffers of the hot-cache transfer plan for one layer."""
    resident: torch.Tensor        # [B, Hkv, slots] int32, -1 = empty
    slot_of_union: torch.Tensor   # [B, Hkv, T*k]
    miss_chunk: torch.Tensor
    miss_slot: torch.Tensor
    miss_count: torch.Tensor      # [B, Hkv]
    hit_count: torch.Tensor

    @staticmethod
    def empty(B, Hkv, T, k, slots, device):
        i32 = dict(dtype=torch.int32, device=device)
        return CachePlan(torch.full((B, Hkv, slots), -1, **i32), torch.empty(B, Hkv, T * k, **i32),
                         torch.empty(B, Hkv, T * k, **i32), torch.empty(B, Hkv, T * k, **i32),
                         torch.empty(B, Hkv, **i32), torch.empty(B, Hkv, **i32))

    def as_c(self) -> dk_cache_plan:
        return dk_cache_plan(self.resident.data_ptr(), self.resident.shape[2],
                             self.slot_of_union.data_ptr(), self.miss_chunk.data_ptr(),
                             self.miss_slot.data_ptr(), self.miss_count.data_ptr(),
                             self.hit_count.data_ptr())


@_on_stream
def union_select(topk_idx: torch.Tensor, C: int, union_ids=None, member=None, count=None,
                 overlap=None, plan: CachePlan | None = None, stream=None):
    B, Hkv, T, k = topk_idx.shape
    _need(topk_idx, torch.int32, (B, Hkv, T, k), "topk_idx")
    dev = topk_idx.device
    if union_ids is None:
        union_ids = torch.empty(B, Hkv, T * k, dtype=torch.int32, device=dev)
    if member is None:
        member = torch.empty(B, Hkv, T * k, dtype=torch.uint8, device=dev)
    if count is None:
        count = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    if overlap is None:
        overlap = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    cplan = ctypes.byref(plan.as_c()) if plan is not None else None
    _check(lib.dk_union_select(_ptr(topk_idx), B, Hkv, T, k, C, _ptr(union_ids), _ptr(member),
                               _ptr(count), _ptr(overlap), cplan, _stream(stream)))
    return union_ids, member, count, overlap


DK_SRC_DEVICE, DK_SRC_HOST_COPY, DK_SRC_HOST_MAPPED = 0, 1, 2


@_on_stream
def gather_kv(K_src, V_src, src_chunk, count, chunk, K_dst, V_dst, dst_slot=None,
              src_blocks=None, dst_blocks=None, stream=None):
    """Copy chunks src_chunk[b, g, j] (j < count[b, g]) into slots of K_dst / V_dst.

    The source kind follows from where the tensors live:
      device pool                          -> one gather kernel;
      pinned host pool, host (CPU) lists   -> hipMemcpyAsync per run of chunks;
      pinned host pool, device lists       -> one gather kernel reading the pool
                                              through its device mapping (zero-copy).
    """
    B, Hkv, L, d = K_src.shape
    N = src_chunk.shape[2]
    host_pool = not K_src.is_cuda
    if host_pool and not (K_src.is_pinned() and V_src.is_pinned()):
        raise ValueError("a host KV pool must be in pinned memory")
    lists_on_host = not src_chunk.is_cuda
    if not host_pool and lists_on_host:
        raise ValueError("a device KV pool needs device lists")
    kind = (DK_SRC_DEVICE if not host_pool else
            DK_SRC_HOST_COPY if lists_on_host else DK_SRC_HOST_MAPPED)
    for name, t in (("src_chunk", src_chunk), ("dst_slot", dst_slot), ("count", count)):
        if t is not None and (t.is_cuda == lists_on_host or t.dtype != torch.int32 or not t.is_contiguous()):
            raise ValueError(f"{name}: int32 contiguous, on the same side as src_chunk")
    if src_blocks is None:
        src_blocks = L // chunk
    if dst_blocks is None:
        dst_blocks = K_dst.shape[2] // chunk
    _check(lib.dk_gather_kv(_ptr(K_src), _ptr(V_src), _dtype(K_src), pool_strides(K_src), B, Hkv,
                            chunk, d, _ptr(src_chunk), _ptr(dst_slot), _ptr(count), N, src_blocks,
                            _ptr(K_dst), _ptr(V_dst), pool_strides(K_dst), dst_blocks, kind,
                            _stream(stream)))
    return kind


def attn_workspace_size(B, Hkv, T, Hq, dv, N, chunk) -> int:
    return int(lib.dk_attn_workspace_size(B, Hkv, T, Hq, dv, N, chunk))


@_on_stream
def sparse_decode_attn(q, K, V, block_ids, member, count, chunk: int, scale: float,
                       pool_blocks: int | None = None, out=None, lse=None, ws=None, want_lse=True,
                       stream=None):
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    dv = V.shape[3]
    N = block_ids.shape[2]
    _need(q, torch.float32, (B, T, Hq, dk), "q")
    _need(block_ids, torch.int32, (B, Hkv, N), "block_ids")
    if member is not None:
        _need(member, torch.uint8, (B, Hkv, N), "member")
    if count is not None:
        _need(count, torch.int32, (B, Hkv), "count")
    if out is None:
        out = torch.empty(B, T, Hq, dv, dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    if pool_blocks is None:
        pool_blocks = K.shape[2] // chunk
    nbytes = attn_workspace_size(B, Hkv, T, Hq, dv, N, chunk)
    if ws is None and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if K.dtype != V.dtype:
        raise ValueError("K and V must share a dtype")
    _check(lib.dk_sparse_decode_attn(_ptr(q), B, T, Hq, Hkv, _ptr(K), _ptr(V), _dtype(K),
                                     pool_strides(K), pool_strides(V), dk, dv, chunk,
                                     _ptr(block_ids), _ptr(member), _ptr(count), N, pool_blocks,
                                     float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))
    return out, lse


def decode_step_workspace_size(B, Hkv, T, Hq, C, d, k, chunk, with_shadow, with_tail=False) -> int:
    return int(lib.dk_decode_step_workspace_size(B, Hkv, T, Hq, C, d, k, chunk, int(bool(with_shadow)),
                                                 int(bool(with_tail))))


def _attn_extra(B, T, Hkv, dk, dv, K, K_tail, V_tail, tail_len, K_new, V_new) -> dk_attn_extra:
    """The dk_attn_extra of the tail rows and the step's own rows, after shape checks."""
    for name, t in (("K_tail", K_tail), ("V_tail", V_tail), ("K_new", K_new), ("V_new", V_new)):
        if t is not None and t.dtype != K.dtype:
            raise ValueError(f"{name} must have the pools' dtype")
    if K_new is not None:
        _need(K_new, K.dtype, (B, T, Hkv, dk), "K_new")
        _need(V_new, K.dtype, (B, T, Hkv, dv), "V_new")
    if tail_len is not None:
        _need(tail_len, torch.int32, (B,), "tail_len")
    zero = dk_strides(0, 0, 0)
    return dk_attn_extra(_ptr(K_tail), _ptr(V_tail),
                         pool_strides(K_tail) if K_tail is not None else zero,
                         pool_strides(V_tail) if V_tail is not None else zero,
                         _ptr(tail_len), K_tail.shape[2] if K_tail is not None else 0,
                         _ptr(K_new), _ptr(V_new))


@_on_stream
def decode_step(q, lm, K, V, chunk: int, k: int, scale: float, reduce: int = DK_REDUCE_MEAN,
                shadow: Shadow | None = None, topk_idx=None, topk_score=None, union_ids=None, member=None,
                count=None, overlap=None, out=None, lse=None, ws=None, want_scores=False, want_lse=True,
                K_tail=None, V_tail=None, tail_len=None, K_new=None, V_new=None, stream=None):
    """score_topk_union then sparse_decode_attn over its union, as one library call
    (dk_decode_step: one fused kernel where the shapes allow it).  With any of K_tail,
    V_tail, K_new, V_new given, the attention is sparse_decode_attn_tail's."""
    B, T, Hq, d = q.shape
    _, Hkv, C, _ = lm.shape
    _need(q, torch.float32, (B, T, Hq, d), "q")
    if K.dtype != V.dtype:
        raise ValueError("K and V must share a dtype")
    dev = q.device
    i32 = dict(dtype=torch.int32, device=dev)
    topk_idx = torch.empty(B, Hkv, T, k, **i32) if topk_idx is None else topk_idx
    if topk_score is None and want_scores:
        topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=dev)
    union_ids = torch.empty(B, Hkv, T * k, **i32) if union_ids is None else union_ids
    member = torch.empty(B, Hkv, T * k, dtype=torch.uint8, device=dev) if member is None else member
    count = torch.empty(B, Hkv, **i32) if count is None else count
    overlap = torch.empty(B, Hkv, **i32) if overlap is None else overlap
    out = torch.empty(B, T, Hq, d, dtype=torch.float32, device=dev) if out is None else out
    if lse is None and want_lse:
        lse = torch.empty(B, T, Hq, dtype=torch.float32, device=dev)
    with_tail = any(t is not None for t in (K_tail, V_tail, K_new, V_new))
    extra = _attn_extra(B, T, Hkv, d, d, K, K_tail, V_tail, tail_len, K_new, V_new) if with_tail else None
    nbytes = decode_step_workspace_size(B, Hkv, T, Hq, C, d, k, chunk, shadow is not None, with_tail)
    if ws is None and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    csh = ctypes.byref(shadow.as_c()) if shadow is not None else None
    _check(lib.dk_decode_step(_ptr(q), B, T, Hq, Hkv, _ptr(lm), _dtype(lm), pool_strides(lm), C, d, k,
                              float(scale), int(reduce), csh, _ptr(K), _ptr(V), _dtype(K), pool_strides(K),
                              pool_strides(V), chunk, ctypes.byref(extra) if extra is not None else None,
                              _ptr(topk_idx), _ptr(topk_score), _ptr(union_ids),
                              _ptr(member), _ptr(count), _ptr(overlap), _ptr(out), _ptr(lse), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return topk_idx, topk_score, union_ids, member, count, overlap, out, lse


@_on_stream
def sparse_decode_attn_noalloc(q, K, V, block_ids, member, count, chunk: int, scale: float,
                               pool_blocks: int | None = None, out=None, lse=None, want_lse=True, stream=None):
    """sparse_decode_attn with the library's fixed device scratch instead of a workspace
    (dk_sparse_decode_attn_noalloc): the C call allocates nothing.  Calls that overlap
    on one device share that scratch and race."""
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    dv = V.shape[3]
    N = block_ids.shape[2]
    _need(q, torch.float32, (B, T, Hq, dk), "q")
    _need(block_ids, torch.int32, (B, Hkv, N), "block_ids")
    if member is not None:
        _need(member, torch.uint8, (B, Hkv, N), "member")
    if count is not None:
        _need(count, torch.int32, (B, Hkv), "count")
    if K.dtype != V.dtype:
        raise ValueError("K and V must share a dtype")
    if out is None:
        out = torch.empty(B, T, Hq, dv, dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    if pool_blocks is None:
        pool_blocks = K.shape[2] // chunk
    _check(lib.dk_sparse_decode_attn_noalloc(_ptr(q), B, T, Hq, Hkv, _ptr(K), _ptr(V), _dtype(K),
                                             pool_strides(K), pool_strides(V), dk, dv, chunk,
                                             _ptr(block_ids), _ptr(member), _ptr(count), N, pool_blocks,
                                             float(scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


@_on_stream
def mla_decode_attn(q, latent, token_ids, member, count, scale: float, dv: int = 512, out=None, lse=None,
                    ws=None, want_lse=True, stream=None):
    """Attention over latent rows [B, Hkv, L, dk]: the key is the whole row, the value
    its first dv columns (the same buffer), token_ids index tokens (chunk = 1)."""
    return sparse_decode_attn(q, latent, latent[..., :dv], token_ids, member, count, 1, scale,
                              pool_blocks=latent.shape[2], out=out, lse=lse, ws=ws, want_lse=want_lse,
                              stream=stream)


# ----------------------------------------------------------------------------
# one layer of the HBM-pool step with buffers allocated once
# ----------------------------------------------------------------------------

def attn_tail_workspace_size(B, Hkv, T, Hq, dv, N, chunk) -> int:
    return int(lib.dk_attn_tail_workspace_size(B, Hkv, T, Hq, dv, N, chunk))


@_on_stream
def sparse_decode_attn_tail(q, K, V, block_ids, member, count, chunk: int, scale: float, K_tail=None,
                            V_tail=None, tail_len=None, K_new=None, V_new=None, pool_blocks: int | None = None,
                            out=None, lse=None, ws=None, stream=None):
    """sparse_decode_attn plus the tail rows [B, Hkv, tail_max, d] (first tail_len[b]
    rows of request b) and the step's own rows K_new, V_new [B, T, Hkv, d] under the
    dual-token causal rule."""
    B, T, Hq, dk = q.shape
    Hkv = K.shape[1]
    dv = V.shape[3]
    N = block_ids.shape[2]
    _need(q, torch.float32, (B, T, Hq, dk), "q")
    _need(block_ids, torch.int32, (B, Hkv, N), "block_ids")
    if member is not None:
        _need(member, torch.uint8, (B, Hkv, N), "member")
    if count is not None:
        _need(count, torch.int32, (B, Hkv), "count")
    extra = _attn_extra(B, T, Hkv, dk, dv, K, K_tail, V_tail, tail_len, K_new, V_new)
    if out is None:
        out = torch.empty(B, T, Hq, dv, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, T, Hq, dtype=torch.float32, device=q.device)
    if pool_blocks is None:
        pool_blocks = K.shape[2] // chunk
    nbytes = attn_tail_workspace_size(B, Hkv, T, Hq, dv, N, chunk)
    if ws is None and nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check(lib.dk_sparse_decode_attn_tail(_ptr(q), B, T, Hq, Hkv, _ptr(K), _ptr(V), _dtype(K),
                                          pool_strides(K), pool_strides(V), dk, dv, chunk, _ptr(block_ids),
                                          _ptr(member), _ptr(count), N, pool_blocks, ctypes.byref(extra),
                                          float(scale), _ptr(out), _ptr(lse), _ptr(ws),
                                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))
    return out, lse


class DecodeStep:
    """Preallocated buffers for score_topk_union -> sparse_decode_attn.

    ``run(q, lm, K, V)`` enqueues the two calls on the current stream and
    returns the output buffers (reused across calls).
    """

    def __init__(self, B, T, Hq, Hkv, d, C, chunk, k, scale, device, reduce=DK_REDUCE_MEAN,
                 want_scores=True, shadow: Shadow | None = None):
        self.B, self.T, self.Hq, self.Hkv, self.d, self.C = B, T, Hq, Hkv, d, C
        self.chunk, self.k, self.scale, self.reduce = chunk, k, scale, reduce
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty(B, Hkv, T, k, **i32)
        self.topk_score = torch.empty(B, Hkv, T, k, dtype=torch.float32, device=device) \
            if want_scores else None
        self.shadow = shadow
        n = score_topk_workspace_size(B, Hkv, T, C, k, shadow is not None)
        self.ws_topk = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        self.union_ids = torch.empty(B, Hkv, T * k, **i32)
        self.member = torch.empty(B, Hkv, T * k, dtype=torch.uint8, device=device)
        self.count = torch.empty(B, Hkv, **i32)
        self.overlap = torch.empty(B, Hkv, **i32)
        n = attn_workspace_size(B, Hkv, T, Hq, d, T * k, chunk)
        self.ws_attn = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
        self.out = torch.empty(B, T, Hq, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(B, T, Hq, dtype=torch.float32, device=device)
        n = decode_step_workspace_size(B, Hkv, T, Hq, C, d, k, chunk, shadow is not None)
        self.ws_step = torch.empty(max(n, 1), dtype=torch.uint8, device=device)

    def run(self, q, lm, K, V, stream=None, fused=False):
        """The two calls, or with fused=True the one dk_decode_step call (same results)."""
        if fused:
            decode_step(q, lm, K, V, self.chunk, self.k, self.scale, self.reduce, self.shadow, self.topk_idx,
                        self.topk_score, self.union_ids, self.member, self.count, self.overlap, self.out,
                        self.lse, self.ws_step, stream=stream)
            return self.out, self.lse
        score_topk_union(q, lm, self.k, self.scale, self.reduce, self.topk_idx, self.topk_score,
                         self.union_ids, self.member, self.count, self.overlap, self.ws_topk,
                         shadow=self.shadow, stream=stream)
        sparse_decode_attn(q, K, V, self.union_ids, self.member, self.count, self.chunk, self.scale,
                           out=self.out, lse=self.lse, ws=self.ws_attn, stream=stream)
        return self.out, self.lse
