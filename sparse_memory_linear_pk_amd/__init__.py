"""Sparse Delta Memory (SDM) layer forward on AMD MI355X (gfx950).

The layer runs in libsdm.so (hand-written HIP kernels: pk_score on MFMA,
pk_topk, sdm_plan and sdm_scan) behind the C ABI in include/sdm.h.  This
module only checks tensor arguments and passes device pointers; PyTorch is used
for device memory and the current HIP stream.

    layer = SDM(B=4, H=1, T=8192, d=2048, S=480, dk=256, k=32, W=64,
                in_bf16=True, state_bf16=False)
    layer.forward(wq, rq, v, alpha, beta, subkeys, mem, out)   # mem updated in place

State tensors ([.., N, d]: the memory, its gradient, a learned initial memory)
may have slot rows mem_stride elements apart (SDM(..., mem_stride=...)): pass
the [.., N, d] view of a [.., N, mem_stride] tensor, as layer.empty_state
allocates it.  SDM.stride_hint gives a stride the scans run faster on.
"""
from __future__ import annotations

import ctypes as C

from ._lib import (SDM_BF16, SDM_F32, Config, SDMError, Timing, check, declared_symbols, lib)

__all__ = ["SDM", "SDMError", "declared_symbols", "lib", "pattern_probe", "pattern_probe_mix"]


def _ptr(t):
    """Device pointer of a tensor (or a raw integer address)."""
    if isinstance(t, int):
        return C.c_void_p(t)
    return C.c_void_p(t.data_ptr())


class SDM:
    """One configured layer (the library handle) bound to a HIP stream."""

    def __init__(self, B, H, T, d, S, dk, k, W, in_bf16=False, state_bf16=False, stream=None, mem_stride=0):
        self.shape = dict(B=B, H=H, T=T, d=d, S=S, dk=dk, k=k, W=W)
        self.in_bf16, self.state_bf16 = bool(in_bf16), bool(state_bf16)
        self.mem_stride = int(mem_stride) or d  # elements from one slot row to the next in state tensors
        self._cfg = Config(B, H, T, d, S, dk, k, W, SDM_BF16 if in_bf16 else SDM_F32,
                           SDM_BF16 if state_bf16 else SDM_F32, int(mem_stride))
        if stream is None:
            import torch
            stream = torch.cuda.current_stream()
        self.stream = stream
        handle = stream if isinstance(stream, int) else stream.cuda_stream
        self._h = C.c_void_p()
        check(lib().sdm_create(C.byref(self._cfg), C.c_void_p(handle), C.byref(self._h)), "sdm_create")

    @classmethod
    def from_config(cls, cfg, stream=None, **overrides):
        kw = dict(B=cfg.B, H=cfg.H, T=cfg.T, d=cfg.d, S=cfg.S, dk=cfg.dk, k=cfg.k, W=cfg.W,
                  in_bf16=cfg.in_bf16, state_bf16=cfg.state_bf16)
        kw.update(overrides)
        return cls(stream=stream, **kw)

    @staticmethod
    def stride_hint(d: int, state_bf16: bool) -> int:
        """sdm_mem_stride_hint: a slot-row stride (elements) the scans run faster on for rows of d values."""
        cfg = Config(1, 1, 1, d, 1, 2, 1, 1, SDM_F32, SDM_BF16 if state_bf16 else SDM_F32, 0)
        return int(lib().sdm_mem_stride_hint(C.byref(cfg)))

    def empty_state(self, *lead, dtype=None, device="cuda"):
        """An uninitialised state tensor [*lead, N, d] whose rows are this layer's mem_stride apart: the
        [..., :d] view of a [*lead, N, mem_stride] allocation.  dtype defaults to the state dtype."""
        import torch
        if dtype is None:
            dtype = torch.bfloat16 if self.state_bf16 else torch.float32
        d, N = self.shape["d"], self.shape["S"] ** 2
        return torch.empty((*lead, N, self.mem_stride), dtype=dtype, device=device)[..., :d]

    # ---- argument checks (shape, dtype, device, contiguity) ------------------
    def _t(self, t, name, shape, dtype, rows=None):
        """Checks a tensor argument; rows (a row stride in elements) allows a [.., N, d] state tensor
        whose rows are that far apart, dense otherwise."""
        if isinstance(t, int):
            return t
        import torch
        want = {"in": torch.bfloat16 if self.in_bf16 else torch.float32,
                "state": torch.bfloat16 if self.state_bf16 else torch.float32,
                "f32": torch.float32, "i32": torch.int32}[dtype]
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != want:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {want}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if rows is not None and rows != shape[-1]:
            want_strides, acc = [], 1
            for n in reversed(tuple(shape[:-1]) + (rows,)):
                want_strides.append(acc)
                acc *= n
            if tuple(t.stride()) != tuple(reversed(want_strides)):
                raise ValueError(f"{name} must be the [..., :{shape[-1]}] view of a contiguous "
                                 f"{tuple(shape[:-1]) + (rows,)} tensor (strides {tuple(t.stride())})")
        elif not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return t

    def _dims(self):
        s = self.shape
        return s["B"], s["H"], s["T"], s["d"], s["S"], s["dk"], s["k"], s["W"]

    def forward(self, wq, rq, v, alpha, beta, subkeys, mem, out):
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(wq, "wq", (B, T, H, dk), "in"), self._t(rq, "rq", (B, T, H, dk), "in"),
                self._t(v, "v", (B, T, H, d), "in"), self._t(alpha, "alpha", (B, T, H), "f32"),
                self._t(beta, "beta", (B, T, H), "f32"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride),
                self._t(out, "out", (B, T, H, d), "f32")]
        check(lib().sdm_forward(self._h, *[_ptr(a) for a in args]), "sdm_forward")

    def step(self, wq, rq, v, alpha, beta, subkeys, mem, out):
        """One token (decode): wq, rq [B, H, dk], v [B, H, d], alpha, beta [B, H], out [B, H, d]."""
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(wq, "wq", (B, H, dk), "in"), self._t(rq, "rq", (B, H, dk), "in"),
                self._t(v, "v", (B, H, d), "in"), self._t(alpha, "alpha", (B, H), "f32"),
                self._t(beta, "beta", (B, H), "f32"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride), self._t(out, "out", (B, H, d), "f32")]
        check(lib().sdm_step(self._h, *[_ptr(a) for a in args]), "sdm_step")

    def forward_train(self, wq, rq, v, alpha, beta, subkeys, mem, out, log):
        """sdm_forward, and every write slot's value before its write into log [B, H, T, W, d] (state dtype)."""
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(wq, "wq", (B, T, H, dk), "in"), self._t(rq, "rq", (B, T, H, dk), "in"),
                self._t(v, "v", (B, T, H, d), "in"), self._t(alpha, "alpha", (B, T, H), "f32"),
                self._t(beta, "beta", (B, T, H), "f32"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride),
                self._t(out, "out", (B, T, H, d), "f32"),
                self._t(log, "log", (B, H, T, W, d), "state")]
        check(lib().sdm_forward_train(self._h, *[_ptr(a) for a in args]), "sdm_forward_train")

    def backward(self, wq, rq, v, alpha, beta, subkeys, mem, log, dout, dmem, dwq, drq, dv, dalpha, dbeta, dsubkeys):
        """Gradients of sdm_forward_train: mem is restored to the initial memory and dmem goes from
        dL/d(final memory) to dL/d(initial memory); the other gradients are written."""
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(wq, "wq", (B, T, H, dk), "in"), self._t(rq, "rq", (B, T, H, dk), "in"),
                self._t(v, "v", (B, T, H, d), "in"), self._t(alpha, "alpha", (B, T, H), "f32"),
                self._t(beta, "beta", (B, T, H), "f32"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride),
                self._t(log, "log", (B, H, T, W, d), "state"),
                self._t(dout, "dout", (B, T, H, d), "f32"),
                self._t(dmem, "dmem", (B, H, S * S, d), "f32", self.mem_stride),
                self._t(dwq, "dwq", (B, T, H, dk), "f32"), self._t(drq, "drq", (B, T, H, dk), "f32"),
                self._t(dv, "dv", (B, T, H, d), "f32"), self._t(dalpha, "dalpha", (B, T, H), "f32"),
                self._t(dbeta, "dbeta", (B, T, H), "f32"),
                self._t(dsubkeys, "dsubkeys", (H, 2, S, dk // 2), "f32")]
        check(lib().sdm_backward(self._h, *[_ptr(a) for a in args]), "sdm_backward")

    def project(self, D, x, w, gate_bias, wq, rq, v, alpha, beta):
        """Input projections: x [B, T, D] bf16, w [H*(2dk+d+2), D] bf16, gate_bias [H, 2] float32 ->
        wq, rq [B, T, H, dk], v [B, T, H, d] (bf16), alpha, beta [B, T, H] (float32)."""
        B, H, T, d, S, dk, k, W = self._dims()
        C_ = 2 * dk + d + 2
        args = [self._t(x, "x", (B, T, D), "in"), self._t(w, "w", (H * C_, D), "in"),
                self._t(gate_bias, "gate_bias", (H, 2), "f32"), self._t(wq, "wq", (B, T, H, dk), "in"),
                self._t(rq, "rq", (B, T, H, dk), "in"), self._t(v, "v", (B, T, H, d), "in"),
                self._t(alpha, "alpha", (B, T, H), "f32"), self._t(beta, "beta", (B, T, H), "f32")]
        check(lib().sdm_project(self._h, int(D), *[_ptr(a) for a in args]), "sdm_project")

    def broadcast_memory(self, m0, mem):
        """mem [B, H, N, d] = B copies of m0 [H, N, d] (state dtype)."""
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(m0, "m0", (H, S * S, d), "state", self.mem_stride),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride)]
        check(lib().sdm_broadcast_memory(self._h, *[_ptr(a) for a in args]), "sdm_broadcast_memory")

    def overlap(self, idx_w, wt_w, idx_r, wt_r, buckets, write_cum, read, queries=None, overlap=None):
        """Bucket-overlap diagnostic of a call's addressing (sdm_overlap): write_cum, read [B, H, T, buckets]
        float32; for int32 query tokens [Q], overlap [B, H, Q, T] float32."""
        B, H, T, d, S, dk, k, W = self._dims()
        R = B * T * H
        args = [self._t(idx_w, "idx_w", (R, W), "i32"), self._t(wt_w, "wt_w", (R, W), "f32"),
                self._t(idx_r, "idx_r", (R, W), "i32"), self._t(wt_r, "wt_r", (R, W), "f32")]
        outs = [self._t(write_cum, "write_cum", (B, H, T, buckets), "f32"),
                self._t(read, "read", (B, H, T, buckets), "f32")]
        Q = 0 if queries is None else int(queries.numel())
        qs = [None, None]
        if Q:
            qs = [self._t(queries, "queries", (Q,), "i32"), self._t(overlap, "overlap", (B, H, Q, T), "f32")]
        check(lib().sdm_overlap(self._h, *[_ptr(a) for a in args], int(buckets), *[_ptr(a) for a in outs], Q,
                                *[None if a is None else _ptr(a) for a in qs]), "sdm_overlap")

    def score(self, q, subkeys, scores):
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(q, "q", (B, T, H, dk), "in"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(scores, "scores", (B * T * H, 2, S), "f32")]
        check(lib().sdm_score(self._h, *[_ptr(a) for a in args]), "sdm_score")

    def select(self, scores, idx, wt):
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(scores, "scores", (B * T * H, 2, S), "f32"), self._t(idx, "idx", (B * T * H, W), "i32"),
                self._t(wt, "wt", (B * T * H, W), "f32")]
        check(lib().sdm_select(self._h, *[_ptr(a) for a in args]), "sdm_select")

    def address(self, q, subkeys, idx, wt):
        B, H, T, d, S, dk, k, W = self._dims()
        args = [self._t(q, "q", (B, T, H, dk), "in"), self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(idx, "idx", (B * T * H, W), "i32"), self._t(wt, "wt", (B * T * H, W), "f32")]
        check(lib().sdm_address(self._h, *[_ptr(a) for a in args]), "sdm_address")

    def address_pair(self, wq, rq, subkeys, idx_w, wt_w, idx_r, wt_r):
        B, H, T, d, S, dk, k, W = self._dims()
        R = B * T * H
        args = [self._t(wq, "wq", (B, T, H, dk), "in"), self._t(rq, "rq", (B, T, H, dk), "in"),
                self._t(subkeys, "subkeys", (H, 2, S, dk // 2), "in"),
                self._t(idx_w, "idx_w", (R, W), "i32"), self._t(wt_w, "wt_w", (R, W), "f32"),
                self._t(idx_r, "idx_r", (R, W), "i32"), self._t(wt_r, "wt_r", (R, W), "f32")]
        check(lib().sdm_address_pair(self._h, *[_ptr(a) for a in args]), "sdm_address_pair")

    def scan_with(self, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, mem, out):
        B, H, T, d, S, dk, k, W = self._dims()
        R = B * T * H
        args = [self._t(idx_w, "idx_w", (R, W), "i32"), self._t(wt_w, "wt_w", (R, W), "f32"),
                self._t(idx_r, "idx_r", (R, W), "i32"), self._t(wt_r, "wt_r", (R, W), "f32"),
                self._t(v, "v", (B, T, H, d), "in"), self._t(alpha, "alpha", (B, T, H), "f32"),
                self._t(beta, "beta", (B, T, H), "f32"),
                self._t(mem, "mem", (B, H, S * S, d), "state", self.mem_stride),
                self._t(out, "out", (B, T, H, d), "f32")]
        check(lib().sdm_scan_with(self._h, *[_ptr(a) for a in args]), "sdm_scan_with")

    # ---- timing ----------------------------------------------------------------
    def set_timing(self, on: bool = True):
        check(lib().sdm_set_timing(self._h, int(on)), "sdm_set_timing")

    def timing(self) -> dict:
        t = Timing()
        check(lib().sdm_get_timing(self._h, C.byref(t)), "sdm_get_timing")
        return {f: getattr(t, f) for f, _ in Timing._fields_}

    @staticmethod
    def workspace_bytes(B, H, T, d, S, dk, k, W, in_bf16=False, state_bf16=False, mem_stride=0) -> int:
        cfg = Config(B, H, T, d, S, dk, k, W, SDM_BF16 if in_bf16 else SDM_F32, SDM_BF16 if state_bf16 else SDM_F32,
                     int(mem_stride))
        n = C.c_size_t()
        check(lib().sdm_workspace_bytes(C.byref(cfg), C.byref(n)), "sdm_workspace_bytes")
        return n.value

    @staticmethod
    def backward_workspace_bytes(B, H, T, d, S, dk, k, W, in_bf16=False, state_bf16=False, mem_stride=0) -> int:
        cfg = Config(B, H, T, d, S, dk, k, W, SDM_BF16 if in_bf16 else SDM_F32, SDM_BF16 if state_bf16 else SDM_F32,
                     int(mem_stride))
        n = C.c_size_t()
        check(lib().sdm_backward_workspace_bytes(C.byref(cfg), C.byref(n)), "sdm_backward_workspace_bytes")
        return n.value

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            check(lib().sdm_destroy(self._h), "sdm_destroy")
            self._h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def pattern_probe(mem, memories: int, rows: int, row_bytes: int, T: int, W: int, seed: int = 0, stream=None):
    """The scan's memory traffic with no arithmetic (sdm_pattern_probe): 3*W*row_bytes*T*memories
    bytes of random 128-byte row segments, two reads per write.  Scrambles mem."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    check(lib().sdm_pattern_probe(_ptr(mem), memories, rows, row_bytes, T, W, seed, C.c_void_p(handle)),
          "sdm_pattern_probe")


def pattern_probe_mix(mem, memories: int, rows: int, row_bytes: int, T: int, W: int, reads: int, writes: int,
                      seed: int = 0, stream=None, row_stride: int = 0):
    """sdm_pattern_probe_mix: (reads + writes)*W*row_bytes*T*memories bytes of random 128-byte row
    segments, reads:writes per slot position and token (2:1 or 4:3), rows row_stride bytes apart
    (0: row_bytes).  Scrambles mem."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    check(lib().sdm_pattern_probe_mix(_ptr(mem), memories, rows, row_bytes, row_stride, T, W, reads, writes, seed,
                                      C.c_void_p(handle)), "sdm_pattern_probe_mix")
