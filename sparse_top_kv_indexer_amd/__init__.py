"""Python binding of libsparsekv.so (the MI355X sparse top-k decode step).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  The functions keep the C names (``sparsekv_score``,
``sparsekv_topk``, ``sparsekv_gather_attend``, ``sparsekv_encode``,
``sparsekv_retrieve``, ...); they take torch tensors that live on the GPU,
check dtype / shape / contiguity, pass ``data_ptr()`` values and torch's
current HIP stream, and raise ``SkvError`` on a non-zero status.  Nothing here
computes on the CPU, and nothing falls back: without the built library every
call raises.

torch is imported before the library is loaded so that the process has a
single HIP runtime (torch's); the library resolves its HIP symbols against it.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparsekv.so")
# the checking build (every call first validates tables, windows and selected
# positions); chosen with SKV_DEBUG=1 in the environment or use_debug_library()
LIB_DEBUG_PATH = os.path.join(_HERE, "libsparsekv_debug.so")

SKV_OK, SKV_EINVAL, SKV_EUNSUPPORTED, SKV_EWORKSPACE, SKV_ELAUNCH = range(5)
SKV_F32, SKV_BF16 = 0, 1
(SKV_OP_SCORE, SKV_OP_TOPK, SKV_OP_GATHER_ATTEND, SKV_OP_ENCODE, SKV_OP_RETRIEVE, SKV_OP_SELECT,
 SKV_OP_SELECT_ATTEND, SKV_OP_BLOCK_SELECT) = range(8)

c_vp, c_i32, c_f32, c_sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t


class SkvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


class skv_kv(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("dtype", ctypes.c_int), ("B", c_i32), ("H", c_i32),
                ("d_k", c_i32), ("d_v", c_i32), ("block", c_i32), ("L_max", c_i32),
                ("block_table", c_vp), ("token_table", c_vp), ("seq_len", c_vp),
                ("n_blocks", c_i32)]


class skv_window(ctypes.Structure):
    _fields_ = [("lo", c_vp), ("hi", c_vp)]


class skv_codebook(ctypes.Structure):
    _fields_ = [("d", c_i32), ("n_sub", c_i32), ("m", c_i32), ("signs", c_vp),
                ("levels", c_f32 * 8), ("thresh", c_f32 * 7)]


class skv_index(ctypes.Structure):
    _fields_ = [("ids", c_vp), ("cw", c_vp), ("hist", c_vp), ("pos", c_vp),
                ("n", c_i32), ("cap", c_i32), ("H", c_i32)]


class skv_retrieve_trace(ctypes.Structure):
    _fields_ = [("votes", c_vp), ("cand", c_vp), ("est", c_vp)]


class skv_move(ctypes.Structure):
    _fields_ = [("b", c_i32), ("t", c_i32), ("src", c_i32), ("dst", c_i32)]


# symbol -> (restype, argtypes)
_SIGS = {
    "sparsekv_score": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, c_vp, c_vp]),
    "sparsekv_topk": (c_i32, [c_vp, c_i32, c_i32, c_i32, skv_window, c_i32, c_vp, c_vp, c_vp,
                              c_sz, c_vp]),
    "sparsekv_select": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window, c_i32, c_vp,
                                c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_score_hist": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window, c_vp, c_vp,
                                    c_sz, c_vp]),
    "sparsekv_topk_resume": (c_i32, [c_vp, c_i32, c_i32, c_i32, skv_window, c_i32, c_vp, c_vp,
                                     c_vp, c_sz, c_vp]),
    "sparsekv_score_prefilter": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window, c_vp,
                                         c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_topk_prefiltered": (c_i32, [c_vp, c_i32, c_i32, c_i32, skv_window, c_i32, c_vp,
                                          c_f32, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_gather_attend": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, c_vp, c_i32,
                                       skv_window, c_f32, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_select_attend": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window, c_i32,
                                       c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_select_attend_resume": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window,
                                              c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                              c_vp]),
    "sparsekv_indexer_attend": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, ctypes.POINTER(skv_kv),
                                        c_vp, c_i32, skv_window, c_i32, c_f32, c_vp, c_vp, c_vp,
                                        c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_segments": (c_i32, [ctypes.POINTER(skv_kv), c_i32, c_i32]),
    "sparsekv_score_segments": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window, c_i32,
                                        c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_select_attend_segments": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window,
                                                c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                                                c_vp]),
    "sparsekv_select_attend_noalloc_bytes": (c_sz, [ctypes.POINTER(skv_kv), c_i32]),
    "sparsekv_select_attend_noalloc": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_i32, skv_window,
                                               c_i32, c_f32, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "sparsekv_block_summary_bytes": (c_sz, [c_i32, c_i32, c_i32]),
    "sparsekv_block_summarize": (c_i32, [ctypes.POINTER(skv_kv), c_i32, c_i32, c_i32, c_vp, c_vp]),
    "sparsekv_block_summarize_last": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_vp]),
    "sparsekv_block_select": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_vp, c_i32, skv_window, c_i32,
                                      c_vp, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_waste_ratio": (ctypes.c_double, [c_vp, c_i32]),
    "sparsekv_compact_plan": (c_i32, [c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_i32,
                                      ctypes.c_double, c_i32, c_vp, ctypes.POINTER(c_i32), c_vp,
                                      ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]),
    "sparsekv_compact_apply": (c_i32, [ctypes.POINTER(skv_kv), c_i32, c_vp, c_i32, c_vp, c_vp]),
    "sparsekv_live_hash": (c_i32, [ctypes.POINTER(skv_kv), c_vp, c_vp, c_vp]),
    "sparsekv_check_unique_ws_bytes": (c_sz, [c_i32]),
    "sparsekv_check_unique": (c_i32, [ctypes.POINTER(skv_kv), c_i32, c_vp, c_vp, c_sz, c_vp]),
    "sparsekv_codebook_init": (c_i32, [c_i32, ctypes.POINTER(c_f32), ctypes.POINTER(c_f32)]),
    "sparsekv_encode": (c_i32, [ctypes.POINTER(skv_codebook), ctypes.POINTER(skv_kv), c_i32,
                                c_i32, c_i32, ctypes.POINTER(skv_index), c_vp]),
    "sparsekv_update_buffer": (c_i32, [ctypes.POINTER(skv_codebook), ctypes.POINTER(skv_kv), c_i32,
                                       c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(skv_index),
                                       ctypes.POINTER(c_i32), c_vp]),
    "sparsekv_retrieve": (c_i32, [ctypes.POINTER(skv_codebook), ctypes.POINTER(skv_index), c_vp,
                                  c_i32, ctypes.c_double, ctypes.c_double, c_i32, c_vp, c_vp,
                                  ctypes.POINTER(skv_retrieve_trace), c_vp, c_sz, c_vp]),
    "sparsekv_workspace_size": (c_sz, [ctypes.c_int, ctypes.POINTER(skv_kv), c_i32, c_i32,
                                       ctypes.POINTER(skv_index)]),
    "sparsekv_retrieve_workspace_size": (c_sz, [ctypes.POINTER(skv_index), c_i32, ctypes.c_double,
                                                c_i32]),
    "sparsekv_validate_ws_bytes": (c_sz, [ctypes.POINTER(skv_kv), c_i32]),
    "sparsekv_validate": (c_i32, [ctypes.POINTER(skv_kv), skv_window, c_vp, c_i32, c_vp, c_vp,
                                  c_sz, c_vp]),
    "sparsekv_debug_status": (c_i32, [ctypes.POINTER(c_i32)]),
    "sparsekv_is_debug_build": (c_i32, []),
    "sparsekv_status_string": (ctypes.c_char_p, [c_i32]),
    "sparsekv_version": (c_i32, []),
}

_lib = None


def _load(path: str):
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (run __graft_entry__.build()); there is no fallback "
                           "path" % os.path.basename(path))
    L = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


def lib():
    """The loaded library (the checking build when SKV_DEBUG=1 is set in the
    environment); raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_DEBUG_PATH if os.environ.get("SKV_DEBUG") == "1" else LIB_PATH)
    return _lib


def use_debug_library(on: bool = True):
    """Route every following call to the checking build (on) or the release
    build; both may be loaded in one process."""
    global _lib
    _lib = _load(LIB_DEBUG_PATH if on else LIB_PATH)
    return _lib


def _check(fn: str, st: int):
    if st != SKV_OK:
        raise SkvError(fn, st, lib().sparsekv_status_string(st).decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t


# ---------------------------------------------------------------------------
@dataclass
class KVTensors:
    """Device-resident KV storage matching skv_kv."""
    k: torch.Tensor
    v: Optional[torch.Tensor]
    dtype: str          # "bf16" | "f32"
    B: int
    H: int
    d_k: int
    d_v: int
    block: int
    L_max: int
    block_table: Optional[torch.Tensor]
    token_table: Optional[torch.Tensor]
    seq_len: torch.Tensor

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def c(self) -> skv_kv:
        td = self.torch_dtype
        _dev(self.k, "k", td)
        if self.v is not None:
            _dev(self.v, "v", td)
        _dev(self.seq_len, "seq_len", torch.int32)
        for nm in ("block_table", "token_table"):
            t = getattr(self, nm)
            if t is not None:
                _dev(t, nm, torch.int32)
        n_blocks = self.k.numel() // (self.H * 16 * self.d_k) if self.block == 16 else 0
        return skv_kv(_ptr(self.k), _ptr(self.v), SKV_BF16 if self.dtype == "bf16" else SKV_F32,
                      self.B, self.H, self.d_k, self.d_v, self.block, self.L_max,
                      _ptr(self.block_table), _ptr(self.token_table), _ptr(self.seq_len),
                      n_blocks)


def to_device(arr: np.ndarray, device, bf16: bool = False) -> torch.Tensor:
    """Host array -> contiguous device tensor (uint16 bf16 bits -> torch.bfloat16)."""
    a = np.ascontiguousarray(arr)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def kv_to_device(kv, device="cuda") -> KVTensors:
    """Upload any object with the skv_kv fields (numpy arrays) to the GPU."""
    bf = kv.dtype == "bf16"
    opt = lambda x: None if x is None else to_device(np.asarray(x, np.int32), device)
    return KVTensors(k=to_device(kv.k, device, bf), v=None if kv.v is None else to_device(kv.v, device, bf),
                     dtype=kv.dtype, B=kv.B, H=kv.H, d_k=kv.d_k, d_v=kv.d_v, block=kv.block,
                     L_max=kv.L_max, block_table=opt(kv.block_table), token_table=opt(kv.token_table),
                     seq_len=opt(kv.seq_len))


# ---------------------------------------------------------------------------
def sparsekv_score(kv: KVTensors, q: torch.Tensor, G: int, scores: Optional[torch.Tensor] = None):
    """scores[b][h][t] = max_g q[b][h*G+g] . K(b,h,t)  (fp32, -inf for dead / past seq_len)."""
    _dev(q, "q", kv.torch_dtype)
    if q.shape != (kv.B, kv.H * G, kv.d_k):
        raise ValueError("q must be [B][H*G][d_k]")
    if scores is None:
        scores = torch.empty((kv.B, kv.H, kv.L_max), dtype=torch.float32, device=q.device)
    _dev(scores, "scores", torch.float32)
    c = kv.c()
    _check("sparsekv_score", lib().sparsekv_score(ctypes.byref(c), _ptr(q), G, _ptr(scores), _stream()))
    return scores


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled device workspace (the library keeps it zero between calls)."""
    return torch.zeros(max(1, int(nbytes)), dtype=torch.uint8, device=device)


def topk_workspace_size(B: int, H: int, L_max: int, k: int) -> int:
    c = skv_kv(None, None, SKV_F32, B, H, 8, 8, 0, L_max, None, None, None)
    return int(lib().sparsekv_workspace_size(SKV_OP_TOPK, ctypes.byref(c), 0, k, None))


def sparsekv_topk(scores: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, k: int,
                  idx: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None):
    """Exact top-k per row, ascending positions, -1 padded; returns (idx, count)."""
    _dev(scores, "scores", torch.float32)
    B, H, L = scores.shape
    _dev(lo, "lo", torch.int32)
    _dev(hi, "hi", torch.int32)
    if idx is None:
        idx = torch.empty((B, H, k), dtype=torch.int32, device=scores.device)
    if count is None:
        count = torch.empty((B, H), dtype=torch.int32, device=scores.device)
    _dev(idx, "idx", torch.int32)
    _dev(count, "count", torch.int32)
    if ws is None:
        ws = workspace(topk_workspace_size(B, H, L, k), scores.device)
    wsz = ws.numel() * ws.element_size()
    _check("sparsekv_topk", lib().sparsekv_topk(_ptr(scores), B, H, L, skv_window(_ptr(lo), _ptr(hi)),
                                                 k, _ptr(idx), _ptr(count), _ptr(ws), wsz, _stream()))
    return idx, count


def sparsekv_select(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor, hi: torch.Tensor,
                    k: int, scores: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                    count: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """Score scan + exact top-k in one call; returns (scores, idx, count)."""
    _dev(q, "q", kv.torch_dtype)
    if q.shape != (kv.B, kv.H * G, kv.d_k):
        raise ValueError("q must be [B][H*G][d_k]")
    dev = q.device
    if scores is None:
        scores = torch.empty((kv.B, kv.H, kv.L_max), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((kv.B, kv.H, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((kv.B, kv.H), dtype=torch.int32, device=dev)
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (lo, "lo", torch.int32), (hi, "hi", torch.int32)):
        _dev(t, nm, dt)
    if ws is None:
        ws = workspace(sparsekv_workspace_size(SKV_OP_SELECT, kv, G, k), dev)
    c = kv.c()
    _check("sparsekv_select",
           lib().sparsekv_select(ctypes.byref(c), _ptr(q), G, skv_window(_ptr(lo), _ptr(hi)), k,
                                 _ptr(scores), _ptr(idx), _ptr(count), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream()))
    return scores, idx, count


def sparsekv_select_attend(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                           hi: torch.Tensor, k: int, scale: float,
                           scores: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                           count: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           ws: Optional[torch.Tensor] = None):
    """One fused decode step (score scan, exact top-k, gather + attention);
    returns (scores, idx, count, out), the results of sparsekv_select followed
    by sparsekv_gather_attend."""
    _dev(q, "q", kv.torch_dtype)
    if q.shape != (kv.B, kv.H * G, kv.d_k):
        raise ValueError("q must be [B][H*G][d_k]")
    dev = q.device
    if scores is None:
        scores = torch.empty((kv.B, kv.H, kv.L_max), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((kv.B, kv.H, k), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((kv.B, kv.H), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((kv.B, kv.H * G, kv.d_v), dtype=torch.float32, device=dev)
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (out, "out", torch.float32),
                      (lo, "lo", torch.int32), (hi, "hi", torch.int32)):
        _dev(t, nm, dt)
    if ws is None:
        ws = workspace(sparsekv_workspace_size(SKV_OP_SELECT_ATTEND, kv, G, k), dev)
    c = kv.c()
    _check("sparsekv_select_attend",
           lib().sparsekv_select_attend(ctypes.byref(c), _ptr(q), G, skv_window(_ptr(lo), _ptr(hi)), k,
                                        float(scale), _ptr(scores), _ptr(idx), _ptr(count), _ptr(out),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return scores, idx, count, out


def sparsekv_select_attend_resume(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                                  hi: torch.Tensor, k: int, scale: float, scores: torch.Tensor,
                                  idx: torch.Tensor, count: torch.Tensor, out: torch.Tensor,
                                  ws: torch.Tensor):
    """The second half of sparsekv_select_attend, after sparsekv_score_hist on ws."""
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (out, "out", torch.float32)):
        _dev(t, nm, dt)
    c = kv.c()
    _check("sparsekv_select_attend_resume",
           lib().sparsekv_select_attend_resume(ctypes.byref(c), _ptr(q), G,
                                               skv_window(_ptr(lo), _ptr(hi)), k, float(scale),
                                               _ptr(scores), _ptr(idx), _ptr(count), _ptr(out),
                                               _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return idx, count, out


def sparsekv_indexer_attend(ikv: KVTensors, iq: torch.Tensor, iG: int, kv: KVTensors,
                            q: torch.Tensor, G: int, lo: torch.Tensor, hi: torch.Tensor, k: int,
                            scale: float, scores: torch.Tensor, idx: torch.Tensor,
                            count: torch.Tensor, out: torch.Tensor, ws: torch.Tensor):
    """The indexer + shared-latent step: the indexer's score scan over ikv,
    the exact top-k, and the latent attention over kv; returns (scores, idx,
    count, out), equal to sparsekv_score_hist + sparsekv_select_attend_resume."""
    _dev(iq, "iq", ikv.torch_dtype)
    _dev(q, "q", kv.torch_dtype)
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (out, "out", torch.float32),
                      (lo, "lo", torch.int32), (hi, "hi", torch.int32)):
        _dev(t, nm, dt)
    ic, c = ikv.c(), kv.c()
    _check("sparsekv_indexer_attend",
           lib().sparsekv_indexer_attend(ctypes.byref(ic), _ptr(iq), iG, ctypes.byref(c), _ptr(q), G,
                                         skv_window(_ptr(lo), _ptr(hi)), k, float(scale),
                                         _ptr(scores), _ptr(idx), _ptr(count), _ptr(out), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream()))
    return scores, idx, count, out


def sparsekv_segments(kv: KVTensors, G: int, k: int) -> int:
    """Scan segments per row of the segment-candidate path for attending
    over kv with G query heads and top-k k (0: the path does not apply)."""
    c = kv.c()
    return int(lib().sparsekv_segments(ctypes.byref(c), G, k))


def sparsekv_score_segments(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                            hi: torch.Tensor, k: int, scores: torch.Tensor, ws: torch.Tensor):
    """sparsekv_score that also lists each row's segment candidates into ws."""
    _dev(q, "q", kv.torch_dtype)
    _dev(scores, "scores", torch.float32)
    c = kv.c()
    _check("sparsekv_score_segments",
           lib().sparsekv_score_segments(ctypes.byref(c), _ptr(q), G, skv_window(_ptr(lo), _ptr(hi)),
                                         k, _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream()))
    return scores


def sparsekv_select_attend_segments(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                                    hi: torch.Tensor, k: int, scale: float, scores: torch.Tensor,
                                    idx: torch.Tensor, count: torch.Tensor, out: torch.Tensor,
                                    ws: torch.Tensor):
    """The selecting half after sparsekv_score_segments on ws."""
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (out, "out", torch.float32)):
        _dev(t, nm, dt)
    c = kv.c()
    _check("sparsekv_select_attend_segments",
           lib().sparsekv_select_attend_segments(ctypes.byref(c), _ptr(q), G,
                                                 skv_window(_ptr(lo), _ptr(hi)), k, float(scale),
                                                 _ptr(scores), _ptr(idx), _ptr(count), _ptr(out),
                                                 _ptr(ws), ws.numel() * ws.element_size(),
                                                 _stream()))
    return idx, count, out


NOALLOC_SCRATCH_BYTES = 16 << 20


def sparsekv_select_attend_noalloc_bytes(kv: KVTensors, G: int) -> int:
    c = kv.c()
    return int(lib().sparsekv_select_attend_noalloc_bytes(ctypes.byref(c), G))


def sparsekv_select_attend_noalloc(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                                   hi: torch.Tensor, k: int, scale: float, scores: torch.Tensor,
                                   idx: torch.Tensor, count: torch.Tensor, out: torch.Tensor):
    """sparsekv_select_attend with the library's own per-GPU scratch instead
    of a workspace; the caller passes every output (nothing is allocated).
    Returns (scores, idx, count, out)."""
    _dev(q, "q", kv.torch_dtype)
    if q.shape != (kv.B, kv.H * G, kv.d_k):
        raise ValueError("q must be [B][H*G][d_k]")
    for t, nm, dt in ((scores, "scores", torch.float32), (idx, "idx", torch.int32),
                      (count, "count", torch.int32), (out, "out", torch.float32),
                      (lo, "lo", torch.int32), (hi, "hi", torch.int32)):
        _dev(t, nm, dt)
    c = kv.c()
    _check("sparsekv_select_attend_noalloc",
           lib().sparsekv_select_attend_noalloc(ctypes.byref(c), _ptr(q), G,
                                                skv_window(_ptr(lo), _ptr(hi)), k, float(scale),
                                                _ptr(scores), _ptr(idx), _ptr(count), _ptr(out),
                                                _stream()))
    return scores, idx, count, out


def sparsekv_block_summary_bytes(n_blocks: int, H: int, d_k: int) -> int:
    return int(lib().sparsekv_block_summary_bytes(n_blocks, H, d_k))


def block_summary_pool(kv: KVTensors) -> torch.Tensor:
    """A summary pool for every physical block of kv's pool (bf16 rows of 2 d_k)."""
    n_blocks = pool_blocks(kv)
    nb = sparsekv_block_summary_bytes(n_blocks, kv.H, kv.d_k)
    return torch.zeros(nb // 2, dtype=torch.bfloat16, device=kv.k.device)


def sparsekv_block_summarize(kv: KVTensors, b: int, j0: int, j1: int, summ: torch.Tensor):
    """(Re)build the min / max summaries of logical blocks [j0, j1) of sequence b."""
    _dev(summ, "summ", torch.bfloat16)
    n_blocks = pool_blocks(kv)
    if summ.numel() * 2 < sparsekv_block_summary_bytes(n_blocks, kv.H, kv.d_k):
        raise ValueError("summ is smaller than the summary pool of kv's blocks")
    c = kv.c()
    _check("sparsekv_block_summarize",
           lib().sparsekv_block_summarize(ctypes.byref(c), b, j0, j1, _ptr(summ), _stream()))
    return summ


def sparsekv_block_summarize_last(kv: KVTensors, summ: torch.Tensor):
    """(Re)build the summary of the block holding each sequence's last token."""
    _dev(summ, "summ", torch.bfloat16)
    n_blocks = pool_blocks(kv)
    if summ.numel() * 2 < sparsekv_block_summary_bytes(n_blocks, kv.H, kv.d_k):
        raise ValueError("summ is smaller than the summary pool of kv's blocks")
    c = kv.c()
    _check("sparsekv_block_summarize_last",
           lib().sparsekv_block_summarize_last(ctypes.byref(c), _ptr(summ), _stream()))
    return summ


def sparsekv_block_select(kv: KVTensors, summ: torch.Tensor, q: torch.Tensor, G: int,
                          lo: torch.Tensor, hi: torch.Tensor, K: int,
                          blk_scores: Optional[torch.Tensor] = None,
                          blk_idx: Optional[torch.Tensor] = None,
                          blk_count: Optional[torch.Tensor] = None,
                          tok_idx: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """Block scores from the summaries, the exact top-K blocks and their
    tokens; returns (blk_scores, blk_idx, blk_count, tok_idx)."""
    _dev(q, "q", kv.torch_dtype)
    _dev(summ, "summ", torch.bfloat16)
    if q.shape != (kv.B, kv.H * G, kv.d_k):
        raise ValueError("q must be [B][H*G][d_k]")
    dev = q.device
    Lb = kv.L_max // 16
    if blk_scores is None:
        blk_scores = torch.empty((kv.B, kv.H, Lb), dtype=torch.float32, device=dev)
    if blk_idx is None:
        blk_idx = torch.empty((kv.B, kv.H, K), dtype=torch.int32, device=dev)
    if blk_count is None:
        blk_count = torch.empty((kv.B, kv.H), dtype=torch.int32, device=dev)
    if tok_idx is None:
        tok_idx = torch.empty((kv.B, kv.H, 16 * K), dtype=torch.int32, device=dev)
    for t, nm, dt, shp in ((blk_scores, "blk_scores", torch.float32, (kv.B, kv.H, Lb)),
                           (blk_idx, "blk_idx", torch.int32, (kv.B, kv.H, K)),
                           (blk_count, "blk_count", torch.int32, (kv.B, kv.H)),
                           (tok_idx, "tok_idx", torch.int32, (kv.B, kv.H, 16 * K))):
        _dev(t, nm, dt)
        if tuple(t.shape) != shp:
            raise ValueError("%s must be %s" % (nm, shp))
    _dev(lo, "lo", torch.int32)
    _dev(hi, "hi", torch.int32)
    if ws is None:
        ws = workspace(sparsekv_workspace_size(SKV_OP_BLOCK_SELECT, kv, G, K), dev)
    c = kv.c()
    _check("sparsekv_block_select",
           lib().sparsekv_block_select(ctypes.byref(c), _ptr(summ), _ptr(q), G,
                                       skv_window(_ptr(lo), _ptr(hi)), K, _ptr(blk_scores),
                                       _ptr(blk_idx), _ptr(blk_count), _ptr(tok_idx), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()))
    return blk_scores, blk_idx, blk_count, tok_idx


def sparsekv_waste_ratio(n_live) -> float:
    a = np.ascontiguousarray(n_live, np.int32)
    return float(lib().sparsekv_waste_ratio(a.ctypes.data_as(c_vp), a.size))


def sparsekv_compact_plan(token_table: np.ndarray, seq_len: np.ndarray, n_blocks: int, b: int,
                          free_blocks, n_free: int, theta_F: float, max_src: int,
                          counts: Optional[np.ndarray] = None):
    """Host-side relocation plan for sequence b.  Returns (moves int32 [n][4]
    = (b, t, src, dst), freed source blocks, number of target blocks)."""
    tt = np.ascontiguousarray(token_table, np.int32)
    sl = np.ascontiguousarray(seq_len, np.int32)
    fb = np.ascontiguousarray(free_blocks, np.int32)
    cn = None if counts is None else np.ascontiguousarray(counts, np.int32)
    B, L = tt.shape
    moves = np.empty((16 * max_src, 4), np.int32)
    src = np.empty(max_src, np.int32)
    nm, ns, nd = c_i32(0), c_i32(0), c_i32(0)
    _check("sparsekv_compact_plan",
           lib().sparsekv_compact_plan(tt.ctypes.data_as(c_vp), sl.ctypes.data_as(c_vp), B, L,
                                       n_blocks, None if cn is None else cn.ctypes.data_as(c_vp),
                                       b, fb.ctypes.data_as(c_vp) if fb.size else None, n_free,
                                       float(theta_F), max_src, moves.ctypes.data_as(c_vp),
                                       ctypes.byref(nm), src.ctypes.data_as(c_vp), ctypes.byref(ns),
                                       ctypes.byref(nd)))
    return moves[: nm.value].copy(), src[: ns.value].copy(), int(nd.value)


def pool_blocks(kv: KVTensors) -> int:
    """Physical 16-token blocks in kv's pool (k is [n_blocks][H][16][d_k])."""
    return kv.k.numel() // (kv.H * 16 * kv.d_k)


def sparsekv_compact_apply(kv: KVTensors, moves: torch.Tensor, err: Optional[torch.Tensor] = None):
    """Copy the moved rows and rewrite kv.token_table (device, in place).
    Moves outside the table or the pool are skipped and counted into err
    (device int32 [1], added to) when it is given."""
    _dev(moves, "moves", torch.int32)
    if moves.dim() != 2 or moves.shape[1] != 4:
        raise ValueError("moves must be int32 [n][4]")
    if err is not None:
        _dev(err, "err", torch.int32)
    c = kv.c()
    _check("sparsekv_compact_apply",
           lib().sparsekv_compact_apply(ctypes.byref(c), pool_blocks(kv), _ptr(moves),
                                        moves.shape[0], _ptr(err), _stream()))


def sparsekv_live_hash(kv: KVTensors, hash_out: Optional[torch.Tensor] = None,
                       count: Optional[torch.Tensor] = None):
    """(hash [B] as int64 bit patterns of the uint64 sums, live count [B])."""
    dev = kv.k.device
    if hash_out is None:
        hash_out = torch.empty(kv.B, dtype=torch.int64, device=dev)
    if count is None:
        count = torch.empty(kv.B, dtype=torch.int32, device=dev)
    _dev(hash_out, "hash", torch.int64)
    _dev(count, "count", torch.int32)
    c = kv.c()
    _check("sparsekv_live_hash",
           lib().sparsekv_live_hash(ctypes.byref(c), _ptr(hash_out), _ptr(count), _stream()))
    return hash_out, count


def sparsekv_check_unique(kv: KVTensors, n_blocks: int, result: Optional[torch.Tensor] = None,
                          ws: Optional[torch.Tensor] = None):
    """I2 check: int32 [2] = (duplicate claims, slots outside the pool)."""
    dev = kv.k.device
    if result is None:
        result = torch.empty(2, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(max(1, int(lib().sparsekv_check_unique_ws_bytes(n_blocks))),
                         dtype=torch.uint8, device=dev)
    c = kv.c()
    _check("sparsekv_check_unique",
           lib().sparsekv_check_unique(ctypes.byref(c), n_blocks, _ptr(result), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()))
    return result


def sparsekv_score_hist(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                        hi: torch.Tensor, scores: torch.Tensor, ws: torch.Tensor):
    """sparsekv_score that also accumulates the top-k key histogram into ws."""
    _dev(q, "q", kv.torch_dtype)
    _dev(scores, "scores", torch.float32)
    c = kv.c()
    _check("sparsekv_score_hist",
           lib().sparsekv_score_hist(ctypes.byref(c), _ptr(q), G, skv_window(_ptr(lo), _ptr(hi)),
                                     _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream()))
    return scores


def sparsekv_topk_resume(scores: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, k: int,
                         idx: torch.Tensor, count: torch.Tensor, ws: torch.Tensor):
    """Finish the exact top-k from the histogram sparsekv_score_hist left in ws."""
    B, H, L = scores.shape
    _check("sparsekv_topk_resume",
           lib().sparsekv_topk_resume(_ptr(scores), B, H, L, skv_window(_ptr(lo), _ptr(hi)), k,
                                      _ptr(idx), _ptr(count), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream()))
    return idx, count


def sparsekv_score_prefilter(kv: KVTensors, q: torch.Tensor, G: int, lo: torch.Tensor,
                             hi: torch.Tensor, thr: torch.Tensor, scores: torch.Tensor,
                             ws: torch.Tensor):
    """sparsekv_score that also lists, per row, the candidates whose score is
    >= thr[b][h] (fp32 [B][H]) into the top-k workspace ws."""
    _dev(q, "q", kv.torch_dtype)
    _dev(scores, "scores", torch.float32)
    _dev(thr, "thr", torch.float32)
    c = kv.c()
    _check("sparsekv_score_prefilter",
           lib().sparsekv_score_prefilter(ctypes.byref(c), _ptr(q), G,
                                          skv_window(_ptr(lo), _ptr(hi)), _ptr(thr), _ptr(scores),
                                          _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return scores


def sparsekv_topk_prefiltered(scores: torch.Tensor, lo: torch.Tensor, hi: torch.Tensor, k: int,
                              thr: torch.Tensor, idx: torch.Tensor, count: torch.Tensor,
                              ws: torch.Tensor, alpha: float = 0.5,
                              used: Optional[torch.Tensor] = None):
    """Exact top-k from the survivors sparsekv_score_prefilter listed in ws
    (the whole row where they do not suffice); thr is updated in place by the
    EMA of the rows' k-th scores.  used[b][h] = 1 where the survivors sufficed."""
    B, H, L = scores.shape
    _dev(thr, "thr", torch.float32)
    _check("sparsekv_topk_prefiltered",
           lib().sparsekv_topk_prefiltered(_ptr(scores), B, H, L, skv_window(_ptr(lo), _ptr(hi)),
                                           k, _ptr(thr), float(alpha), _ptr(idx), _ptr(count),
                                           _ptr(used) if used is not None else None, _ptr(ws),
                                           ws.numel() * ws.element_size(), _stream()))
    return idx, count


def sparsekv_workspace_size(op: int, kv: Optional[KVTensors], G: int, k: int, index=None) -> int:
    c = kv.c() if kv is not None else None
    return int(lib().sparsekv_workspace_size(op, ctypes.byref(c) if c is not None else None, G, k,
                                             ctypes.byref(index) if index is not None else None))


def sparsekv_gather_attend(kv: KVTensors, q: torch.Tensor, G: int, idx: Optional[torch.Tensor], k: int,
                           lo: torch.Tensor, hi: torch.Tensor, scale: float,
                           out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """out[b][h*G+g] = softmax attention over selected + sink + local (fp32)."""
    _dev(q, "q", kv.torch_dtype)
    if idx is not None:
        _dev(idx, "idx", torch.int32)
    if out is None:
        out = torch.empty((kv.B, kv.H * G, kv.d_v), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32)
    if ws is None:
        ws = workspace(sparsekv_workspace_size(SKV_OP_GATHER_ATTEND, kv, G, k), q.device)
    c = kv.c()
    _check("sparsekv_gather_attend",
           lib().sparsekv_gather_attend(ctypes.byref(c), _ptr(q), G, _ptr(idx), k,
                                        skv_window(_ptr(lo), _ptr(hi)), float(scale), _ptr(out),
                                        _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return out


SKV_FLAG_BAD_SEQ_LEN, SKV_FLAG_BAD_WINDOW, SKV_FLAG_BAD_SLOT = 1, 2, 4
SKV_FLAG_DUP_SLOT, SKV_FLAG_BAD_IDX, SKV_FLAG_DUP_IDX = 8, 16, 32


def sparsekv_validate(kv: KVTensors, lo: Optional[torch.Tensor] = None,
                      hi: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                      flags: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The checks of the device-resident tables, windows and selected
    positions; returns the device int32 [1] flag word (OR-ed into flags when
    given, else a zeroed one)."""
    dev = kv.seq_len.device
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device=dev)
    _dev(flags, "flags", torch.int32)
    k = 0
    if idx is not None:
        _dev(idx, "idx", torch.int32)
        k = idx.shape[-1]
    c = kv.c()
    ws = torch.empty(max(1, int(lib().sparsekv_validate_ws_bytes(ctypes.byref(c), k))),
                     dtype=torch.uint8, device=dev)
    _check("sparsekv_validate",
           lib().sparsekv_validate(ctypes.byref(c), skv_window(_ptr(lo), _ptr(hi)), _ptr(idx), k,
                                   _ptr(flags), _ptr(ws), ws.numel(), _stream()))
    return flags


def sparsekv_debug_status() -> int:
    """The checking build's flag word (then cleared); SkvError in release builds."""
    f = c_i32(0)
    _check("sparsekv_debug_status", lib().sparsekv_debug_status(ctypes.byref(f)))
    return int(f.value)


def sparsekv_is_debug_build() -> bool:
    return bool(lib().sparsekv_is_debug_build())


def sparsekv_codebook_init(m: int):
    """(levels[8], thresh[7]) as float32 numpy arrays, from the library's own
    Lloyd-Max derivation (host only)."""
    lv = (c_f32 * 8)()
    th = (c_f32 * 7)()
    _check("sparsekv_codebook_init", lib().sparsekv_codebook_init(m, lv, th))
    return np.array(lv[:], np.float32), np.array(th[:], np.float32)


def sparsekv_status_string(s: int) -> str:
    return lib().sparsekv_status_string(s).decode()


def sparsekv_version() -> int:
    return int(lib().sparsekv_version())


# ------------------------------------------------------------ retrieval ----
@dataclass
class IndexTensors:
    """Device arrays of a compressed-code index (skv_index)."""
    ids: torch.Tensor     # uint8 [H][cap][n_sub]
    cw: torch.Tensor      # int32 [H][cap][n_sub][2]: codes word, then w (fp32 bits)
    hist: torch.Tensor    # int32 [H][n_sub][256]
    pos: torch.Tensor     # int32 [cap]
    n: int
    cap: int
    H: int

    @property
    def codes(self) -> torch.Tensor:
        """A copy of the 4-bit codes as uint8 [H][cap][d/2] (coordinate 2c in
        the low nibble of byte c)."""
        H, cap, n_sub, _ = self.cw.shape
        return self.cw[..., 0].contiguous().view(torch.uint8).reshape(H, cap, 4 * n_sub)

    @property
    def w(self) -> torch.Tensor:
        """A copy of the correction weights as float32 [H][cap][n_sub]."""
        return self.cw[..., 1].contiguous().view(torch.float32)

    def c(self) -> skv_index:
        for t, nm in ((self.ids, "ids"), (self.cw, "cw"), (self.hist, "hist"), (self.pos, "pos")):
            _dev(t, nm)
        return skv_index(_ptr(self.ids), _ptr(self.cw), _ptr(self.hist), _ptr(self.pos), self.n,
                         self.cap, self.H)


def new_index(H: int, cap: int, d: int = 128, n_sub: int = 16, device="cuda") -> IndexTensors:
    """An empty index (histogram zeroed) with room for `cap` entries per head."""
    return IndexTensors(ids=torch.empty((H, cap, n_sub), dtype=torch.uint8, device=device),
                        cw=torch.empty((H, cap, n_sub, 2), dtype=torch.int32, device=device),
                        hist=torch.zeros((H, n_sub, 256), dtype=torch.int32, device=device),
                        pos=torch.empty((cap,), dtype=torch.int32, device=device),
                        n=0, cap=cap, H=H)


@dataclass
class Codebook:
    signs: torch.Tensor   # int8 [d] on the GPU
    levels: np.ndarray    # float32 [8]
    thresh: np.ndarray    # float32 [7]
    d: int = 128
    n_sub: int = 16
    m: int = 8

    def c(self) -> skv_codebook:
        _dev(self.signs, "signs", torch.int8)
        cb = skv_codebook(self.d, self.n_sub, self.m, _ptr(self.signs))
        for i in range(8):
            cb.levels[i] = float(self.levels[i])
        for i in range(7):
            cb.thresh[i] = float(self.thresh[i])
        return cb


def new_codebook(signs: torch.Tensor, d: int = 128, n_sub: int = 16) -> Codebook:
    """Codebook with the library's own Lloyd-Max levels for m = d / n_sub."""
    lv, th = sparsekv_codebook_init(d // n_sub)
    return Codebook(signs=signs, levels=lv, thresh=th, d=d, n_sub=n_sub, m=d // n_sub)


def sparsekv_encode(cb: Codebook, kv: KVTensors, b: int, t0: int, t1: int, index: IndexTensors):
    """Append the keys at logical positions [t0, t1) of sequence b to the index."""
    c = cb.c()
    kc = kv.c()
    ic = index.c()
    _check("sparsekv_encode", lib().sparsekv_encode(ctypes.byref(c), ctypes.byref(kc), b, t0, t1,
                                                     ctypes.byref(ic), _stream()))
    index.n = ic.n
    return index


def sparsekv_update_buffer(cb: Codebook, kv: KVTensors, b: int, seq_len: int, sink: int,
                           local: int, update: int, index: IndexTensors) -> int:
    """Apply the update-buffer rule after appends (seq_len = the sequence's new
    length, already in kv.seq_len[b] on the device); returns the number of
    buffers flushed into the index."""
    c = cb.c()
    kc = kv.c()
    ic = index.c()
    f = c_i32(0)
    _check("sparsekv_update_buffer",
           lib().sparsekv_update_buffer(ctypes.byref(c), ctypes.byref(kc), b, seq_len, sink, local,
                                        update, ctypes.byref(ic), ctypes.byref(f), _stream()))
    index.n = ic.n
    return int(f.value)


def sparsekv_retrieve(cb: Codebook, index: IndexTensors, q: torch.Tensor, G: int, rho: float,
                      beta: float, k_final: int, idx: Optional[torch.Tensor] = None,
                      n_cand: Optional[torch.Tensor] = None, trace: bool = False,
                      ws: Optional[torch.Tensor] = None):
    """Returns (idx [H][k_final] logical ids, n_cand [H], trace dict or None)."""
    _dev(q, "q", torch.bfloat16)
    dev = q.device
    H = index.H
    if idx is None:
        idx = torch.empty((H, k_final), dtype=torch.int32, device=dev)
    if n_cand is None:
        n_cand = torch.empty((H,), dtype=torch.int32, device=dev)
    ic = index.c()
    if ws is None:
        ws = workspace(lib().sparsekv_retrieve_workspace_size(ctypes.byref(ic), G, float(beta),
                                                              k_final), dev)
    tr = None
    trc = None
    if trace:
        C = max(1, min(index.n, int(math.ceil(float(beta) * index.n))))
        tr = {"votes": torch.empty((H, index.n), dtype=torch.uint8, device=dev),
              "cand": torch.empty((H, C), dtype=torch.int32, device=dev),
              "est": torch.empty((H, C), dtype=torch.float32, device=dev)}
        trc = skv_retrieve_trace(_ptr(tr["votes"]), _ptr(tr["cand"]), _ptr(tr["est"]))
    c = cb.c()
    _check("sparsekv_retrieve",
           lib().sparsekv_retrieve(ctypes.byref(c), ctypes.byref(ic), _ptr(q), G, float(rho),
                                   float(beta), k_final, _ptr(idx), _ptr(n_cand),
                                   ctypes.byref(trc) if trc is not None else None, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream()))
    return idx, n_cand, tr


def retrieve_workspace_size(index: IndexTensors, G: int, beta: float, k_final: int) -> int:
    ic = index.c()
    return int(lib().sparsekv_retrieve_workspace_size(ctypes.byref(ic), G, float(beta), k_final))
