"""Binding of libskv_yardstick.so, the streaming-read yardstick beside the
decode-step library (not part of it): argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskv_yardstick.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libskv_yardstick.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.skv_read_probe.restype = ctypes.c_int32
        L.skv_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.skv_read_probe_ex.restype = ctypes.c_int32
        L.skv_read_probe_ex.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.skv_read_pieces.restype = ctypes.c_int32
        L.skv_read_pieces.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def read_probe(buf: torch.Tensor, n_wg: int, sink: Optional[torch.Tensor] = None,
               nontemporal: bool = False) -> torch.Tensor:
    """Read buf once (device, contiguous); returns the sink words [n_wg]."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(n_wg, dtype=torch.int32, device=buf.device)
    st = lib().skv_read_probe_ex(ctypes.c_void_p(buf.data_ptr()),
                                 buf.numel() * buf.element_size(), n_wg, int(nontemporal),
                                 ctypes.c_void_p(sink.data_ptr()),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError("skv_read_probe_ex failed with status %d" % st)
    return sink


def read_pieces(buf: torch.Tensor, order: torch.Tensor, n_wg: int,
                sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read buf's 4 KB pieces in the order order (device int32 piece indices)."""
    if not buf.is_cuda or not buf.is_contiguous() or order.dtype != torch.int32:
        raise ValueError("buf: contiguous GPU tensor; order: GPU int32")
    n = order.numel()
    if buf.numel() * buf.element_size() < 4096 * n:
        raise ValueError("buf holds fewer than len(order) pieces of 4 KB")
    if sink is None:
        sink = torch.empty(n_wg, dtype=torch.int32, device=buf.device)
    st = lib().skv_read_pieces(ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(order.data_ptr()),
                               n, n_wg, ctypes.c_void_p(sink.data_ptr()),
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError("skv_read_pieces failed with status %d" % st)
    return sink
