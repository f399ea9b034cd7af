"""ctypes binding of libspecsam_harness.so: the synthetic target model's logit
boost and memory-system microbenchmarks used by tests and bench.py. Not part
of the verification or drafting path."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
HARNESS_PATH = os.path.join(_PKG, "libspecsam_harness.so")
_h = None


def lib():
    global _h
    if _h is None:
        if not os.path.exists(HARNESS_PATH):
            raise RuntimeError(f"{HARNESS_PATH} is missing: build it with "
                               "`python -m sam_drafting_lossless_amd.build`")
        L = ctypes.CDLL(HARNESS_PATH)
        P, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.hs_boost_step.argtypes = [P, i32, i32, i32, i32, P, i32, P, P, P, P,
                                    P, P, f32, P]
        L.hs_boost_step.restype = i32
        L.hs_read_bw.argtypes = [P, sz, P, i32, P]
        L.hs_read_bw.restype = i32
        L.hs_copy.argtypes = [P, P, sz, P]
        L.hs_copy.restype = i32
        _h = L
    return _h


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class Booster:
    """Applies the synthetic target model's boost to ring slots of noise.

    gt: [B, L] int32 device tensor (token streams); n0: committed lengths at
    step 0. Each call to ``step(slot_tensor, slot_index, nem_prev)`` first adds
    the previous step's emitted counts to the committed lengths, restores what
    this ring slot was boosted with when it was last used, then boosts
    gt[b, n_b + j] in every row j.
    """

    def __init__(self, gt: torch.Tensor, n0, R: int, V: int, nslots: int,
                 boost: float, dtype: int, mask=None):
        B = gt.shape[0]
        dev = gt.device
        self.B, self.R, self.V, self.boost, self.dtype = B, R, V, boost, dtype
        self.gt = gt.contiguous()
        n0 = torch.as_tensor(n0, dtype=torch.int32, device=dev)
        self.ncommit = [n0.clone(), n0.clone()]  # ping-pong
        self.calls = 0
        self.saved_pos = torch.full((nslots, B, R), -1, dtype=torch.int32,
                                    device=dev)
        self.saved_val = torch.zeros((nslots, B, R), dtype=torch.float32,
                                     device=dev)
        self.mask = mask  # optional [steps, B, R] uint8

    def step(self, slot: torch.Tensor, slot_index: int, nem_prev=None,
             step_index: int | None = None, stream=None):
        m = None
        if self.mask is not None and step_index is not None:
            m = self.mask[step_index].data_ptr()
        nin = self.ncommit[self.calls % 2]
        nout = self.ncommit[(self.calls + 1) % 2]
        self.calls += 1
        rc = lib().hs_boost_step(
            slot.data_ptr(), self.dtype, self.B, self.R, self.V,
            self.gt.data_ptr(), self.gt.shape[1], nin.data_ptr(), nout.data_ptr(),
            None if nem_prev is None else nem_prev.data_ptr(),
            self.saved_pos[slot_index].data_ptr(),
            self.saved_val[slot_index].data_ptr(), m, float(self.boost), _s(stream))
        if rc != 0:
            raise RuntimeError(f"hs_boost_step failed ({rc})")


def read_bw(buf: torch.Tensor, sink: torch.Tensor, grid: int = 0, stream=None):
    rc = lib().hs_read_bw(buf.data_ptr(), buf.numel() * buf.element_size(),
                          sink.data_ptr(), grid, _s(stream))
    if rc != 0:
        raise RuntimeError(f"hs_read_bw failed ({rc})")


def copy(dst: torch.Tensor, src: torch.Tensor, stream=None):
    rc = lib().hs_copy(dst.data_ptr(), src.data_ptr(),
                       src.numel() * src.element_size(), _s(stream))
    if rc != 0:
        raise RuntimeError(f"hs_copy failed ({rc})")
