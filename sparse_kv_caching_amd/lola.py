"""ctypes binding of ``include/lola.h`` (``liblola.so``).

Argument marshalling only: every step of the method runs in the HIP library.
torch tensors provide device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``).  There is no fallback: if the
library is missing this module raises on first use.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblola.so")

LOLA_OK = 0
LOLA_ERR_INVALID_ARG = 1
LOLA_ERR_UNSUPPORTED = 2
LOLA_ERR_OUT_OF_MEMORY = 3
LOLA_ERR_HIP = 4
LOLA_ERR_STATE = 5
LOLA_ERR_WORKSPACE = 6
LOLA_DTYPE_F32 = 0
LOLA_DTYPE_BF16 = 1
KERNELS = ("phi", "chain", "attn", "finalize", "decode", "overlap")
READ_STATE, READ_CACHE, READ_WINDOW, READ_ALL = 1, 2, 4, 7   # lola_set_read_branches bits
READ_BEFORE_UPDATE, READ_AFTER_UPDATE = 0, 1                 # lola_set_read_order
DEBUG_SPIN_LIMIT, DEBUG_CHAIN_FAIL_AT, DEBUG_OVERLAP, DEBUG_CHAIN_SPLIT = 0, 1, 2, 3  # lola_debug_set keys
DEBUG_CHAIN_WORKGROUPS = 4
SCORE_SRE, SCORE_KERNEL_SQ, SCORE_KERNEL_ABS, SCORE_KERNEL_RATIO, SCORE_LOCAL_ATTN = range(5)

EXPORTED = [
    "lola_state_init", "lola_state_free", "lola_state_tokens", "lola_prefill_workspace_bytes",
    "lola_prefill_chunk", "lola_prefill_debug", "lola_decode_step", "lola_state_reset",
    "lola_state_check", "lola_profile", "lola_state_export", "lola_state_import",
    "lola_strerror", "lola_last_error",
]


class LolaConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "q_heads", "kv_heads", "head_dim", "feat_half", "window", "cache",
                 "dtype")]


class LolaStateView(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("H", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("win_k", ctypes.c_void_p), ("win_v", ctypes.c_void_p),
                ("cache_pos", ctypes.c_void_p), ("cache_k", ctypes.c_void_p),
                ("cache_v", ctypes.c_void_p)]


class LolaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__("%s failed: %s (%d): %s" % (where, _errname(code), code, detail))
        self.code = code


def _errname(code):
    return {0: "OK", 1: "INVALID_ARG", 2: "UNSUPPORTED", 3: "OUT_OF_MEMORY", 4: "HIP",
            5: "STATE", 6: "WORKSPACE"}.get(code, "UNKNOWN")


_lib = None


def library() -> ctypes.CDLL:
    """Load liblola.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("liblola.so not found at %s: build it first "
                               "(python -m sparse_kv_caching_amd.build)" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        lib.lola_state_init.argtypes = [ctypes.POINTER(LolaConfig), vp, vp, ctypes.POINTER(vp)]
        lib.lola_state_free.argtypes = [vp]
        lib.lola_state_tokens.argtypes = [vp]
        lib.lola_state_tokens.restype = i64
        lib.lola_prefill_workspace_bytes.argtypes = [vp, i32, i32, ctypes.POINTER(sz)]
        lib.lola_prefill_chunk.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, sz, vp]
        lib.lola_prefill_debug.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, sz, vp, vp, vp]
        lib.lola_decode_step.argtypes = [vp, vp, vp, vp, vp, i32, vp]
        lib.lola_state_reset.argtypes = [vp, vp]
        lib.lola_state_check.argtypes = [vp, vp]
        lib.lola_profile.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_longlong)]
        lib.lola_state_export.argtypes = [vp, ctypes.POINTER(LolaStateView), vp]
        lib.lola_state_import.argtypes = [vp, ctypes.POINTER(LolaStateView), vp]
        lib.lola_set_read_branches.argtypes = [vp, i32]
        lib.lola_prefill_sre_map.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp, sz, vp, vp, vp]
        lib.lola_set_read_order.argtypes = [vp, i32]
        lib.lola_state_import_sequence.argtypes = [vp, i32, ctypes.POINTER(LolaStateView), vp]
        lib.lola_state_export_sequence.argtypes = [vp, i32, ctypes.POINTER(LolaStateView), vp]
        lib.lola_state_positions.argtypes = [vp, ctypes.POINTER(i64)]
        lib.lola_debug_set.argtypes = [vp, i32, ctypes.c_longlong]
        lib.lola_set_scoring.argtypes = [vp, i32]
        lib.lola_prefill_chunk_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, i32, vp]
        lib.lola_strerror.argtypes = [i32]
        lib.lola_strerror.restype = ctypes.c_char_p
        lib.lola_last_error.restype = ctypes.c_char_p
        for f in ("lola_state_init", "lola_state_free", "lola_prefill_workspace_bytes",
                  "lola_prefill_chunk", "lola_prefill_debug", "lola_decode_step",
                  "lola_state_reset", "lola_state_check", "lola_profile", "lola_state_export",
                  "lola_state_import", "lola_set_read_branches", "lola_set_read_order",
                  "lola_state_import_sequence", "lola_state_export_sequence",
                  "lola_state_positions", "lola_prefill_sre_map", "lola_debug_set",
                  "lola_prefill_chunk_noalloc", "lola_set_scoring"):
            getattr(lib, f).restype = i32
        _lib = lib
    return _lib


def _check(code: int, where: str):
    if code != LOLA_OK:
        raise LolaError(code, where, library().lola_last_error().decode())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor")
    return ctypes.c_void_p(t.data_ptr())


class LolaLayer:
    """One layer's LoLA state on the current device.

    dtype: torch.bfloat16 or torch.float32 (of q, k, v, W and the stored K/V).
    W: (Hkv, d, m) feature-map weights, copied into the state."""

    def __init__(self, *, batch: int, q_heads: int, kv_heads: int, head_dim: int,
                 window: int, cache: int, W: torch.Tensor, feat_half: int = 64,
                 dtype: torch.dtype = torch.bfloat16, stream=None):
        self.lib = library()
        self.dtype = dtype
        self.cfg = LolaConfig(batch, q_heads, kv_heads, head_dim, feat_half, window, cache,
                              LOLA_DTYPE_BF16 if dtype == torch.bfloat16 else LOLA_DTYPE_F32)
        if W.dtype != dtype:
            raise ValueError("W must have the state dtype")
        self.B, self.Hq, self.Hkv, self.d = batch, q_heads, kv_heads, head_dim
        self.eta, self.lam, self.m = window, cache, feat_half
        self.U = batch * kv_heads
        self._st = ctypes.c_void_p()
        _check(self.lib.lola_state_init(ctypes.byref(self.cfg), _ptr(W), _stream(stream),
                                        ctypes.byref(self._st)), "lola_state_init")

    # -------------------------------------------------------------- lifetime
    def free(self):
        if self._st:
            self.lib.lola_state_free(self._st)
            self._st = ctypes.c_void_p()

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def check(self, stream=None):
        """Synchronise and raise if a kernel recorded a device-side fault."""
        _check(self.lib.lola_state_check(self._st, _stream(stream)), "lola_state_check")

    def reset(self, stream=None):
        """Empty the state (n = 0) without reallocating."""
        _check(self.lib.lola_state_reset(self._st, _stream(stream)), "lola_state_reset")

    def set_read_branches(self, branches: int):
        """Read-branch mask of the following calls: bits READ_STATE (1),
        READ_CACHE (2), READ_WINDOW (4, required); updates are unaffected."""
        _check(self.lib.lola_set_read_branches(self._st, int(branches)), "lola_set_read_branches")

    def set_read_order(self, order: int):
        """READ_BEFORE_UPDATE (0, the chunk schedule) or READ_AFTER_UPDATE (1,
        the literal token recurrence; decode and C = 1 prefill only)."""
        _check(self.lib.lola_set_read_order(self._st, int(order)), "lola_set_read_order")

    def set_scoring(self, rule: int):
        """Cache scoring rule (SCORE_*) of a state holding no token yet."""
        _check(self.lib.lola_set_scoring(self._st, int(rule)), "lola_set_scoring")

    def debug_set(self, key: int, value: int):
        """lola_debug_set: DEBUG_SPIN_LIMIT (exchange polls before a partner
        counts as lost; 0 = default), DEBUG_CHAIN_FAIL_AT (exchange step at
        which the chain gives up; -1 = never), DEBUG_OVERLAP (prefill
        schedule: -1 auto, 0 chain then read, 1 read beside the chain) or
        DEBUG_CHAIN_SPLIT (the chain's workgroups: -1 auto, 0 column slabs x
        candidate groups, 1 candidate groups holding all of H) or
        DEBUG_CHAIN_WORKGROUPS (the chain's workgroups per unit; 0 auto)."""
        _check(self.lib.lola_debug_set(self._st, int(key), int(value)), "lola_debug_set")

    def profile(self, enable: bool):
        """Return {kernel: (ms, launches)} accumulated since the last call and
        switch per-kernel event timing on or off."""
        ms = (ctypes.c_double * len(KERNELS))()
        cnt = (ctypes.c_longlong * len(KERNELS))()
        _check(self.lib.lola_profile(self._st, int(enable), ms, cnt), "lola_profile")
        return {k: (ms[i], cnt[i]) for i, k in enumerate(KERNELS)}

    @property
    def n(self) -> int:
        return int(self.lib.lola_state_tokens(self._st))

    # ---------------------------------------------------------------- compute
    def workspace_bytes(self, T: int, C: int) -> int:
        b = ctypes.c_size_t()
        _check(self.lib.lola_prefill_workspace_bytes(self._st, T, C, ctypes.byref(b)),
               "lola_prefill_workspace_bytes")
        return int(b.value)

    def prefill(self, q, k, v, C: int, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """q (B, Hq, T, d), k, v (B, Hkv, T, d) -> out (B, Hq, T, d) float32."""
        T = q.shape[2]
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        wsp, wsb = ctypes.c_void_p(), 0
        if ws is not None:
            wsp, wsb = _ptr(ws), ws.numel() * ws.element_size()
        _check(self.lib.lola_prefill_chunk(self._st, _ptr(q), _ptr(k), _ptr(v), T, C, _ptr(out),
                                           LOLA_DTYPE_F32, wsp, wsb, _stream(stream)),
               "lola_prefill_chunk")
        return out

    def prefill_noalloc(self, q, k, v, C: int, out: torch.Tensor, stream=None) -> torch.Tensor:
        """lola_prefill_chunk_noalloc: prefill with the library's static
        workspace (no device allocation by the library); out preallocated."""
        T = q.shape[2]
        _check(self.lib.lola_prefill_chunk_noalloc(self._st, _ptr(q), _ptr(k), _ptr(v), T, C,
                                                   _ptr(out), LOLA_DTYPE_F32, _stream(stream)),
               "lola_prefill_chunk_noalloc")
        return out

    def prefill_debug(self, q, k, v, C: int, stream=None):
        """prefill plus the per-chunk record: returns (out, snap_pos (U, nch,
        lam) int32, cand_keys (U, nch, lam + C) int64 holding uint64 bits)."""
        T = q.shape[2]
        nch = (T + C - 1) // C
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        sp = torch.full((self.U, nch, max(self.lam, 1)), -1, dtype=torch.int32, device=q.device)
        ck = torch.zeros((self.U, nch, self.lam + C), dtype=torch.int64, device=q.device)
        _check(self.lib.lola_prefill_debug(self._st, _ptr(q), _ptr(k), _ptr(v), T, C, _ptr(out),
                                           LOLA_DTYPE_F32, ctypes.c_void_p(), 0, _ptr(sp),
                                           _ptr(ck), _stream(stream)), "lola_prefill_debug")
        return out, sp, ck

    def prefill_sre_map(self, q, k, v, C: int, stream=None):
        """prefill plus the SRE diagnostics: returns (y, sre_map (U, nch, T)
        float32, fold_chunk (U, T) int32); see lola_prefill_sre_map."""
        B, Hq, T, d = q.shape
        nch = (T + C - 1) // C
        out = torch.empty((B, Hq, T, d), dtype=torch.float32, device=q.device)
        m = torch.empty((self.U, nch, T), dtype=torch.float32, device=q.device)
        fold = torch.empty((self.U, T), dtype=torch.int32, device=q.device)
        _check(self.lib.lola_prefill_sre_map(self._st, _ptr(q), _ptr(k), _ptr(v), T, C, _ptr(out),
                                             LOLA_DTYPE_F32, None, 0, _ptr(m), _ptr(fold),
                                             _stream(stream)), "lola_prefill_sre_map")
        return out, m, fold

    def decode(self, q, k, v, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """q (B, Hq, d), k, v (B, Hkv, d) -> out (B, Hq, d) float32."""
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        _check(self.lib.lola_decode_step(self._st, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                         LOLA_DTYPE_F32, _stream(stream)), "lola_decode_step")
        return out

    # ------------------------------------------------------ export / import
    def _view_tensors(self, device, units: Optional[int] = None) -> Dict[str, torch.Tensor]:
        U, d, D, lam, eta = units or self.U, self.d, 2 * self.m, self.lam, self.eta
        f = dict(device=device)
        return dict(H=torch.zeros((U, D, d), dtype=torch.float32, **f),
                    s=torch.zeros((U, D), dtype=torch.float32, **f),
                    win_k=torch.zeros((U, max(eta, 1), d), dtype=self.dtype, **f),
                    win_v=torch.zeros((U, max(eta, 1), d), dtype=self.dtype, **f),
                    cache_pos=torch.zeros((U, max(lam, 1)), dtype=torch.int32, **f),
                    cache_k=torch.zeros((U, max(lam, 1), d), dtype=self.dtype, **f),
                    cache_v=torch.zeros((U, max(lam, 1), d), dtype=self.dtype, **f))

    def export(self, stream=None) -> Dict[str, torch.Tensor]:
        """Canonical state: H (U, D, d), s (U, D), win_k/v (U, eta, d) oldest
        first, cache_pos (U, lam) ascending (-1 padding), cache_k/v.  Raises if
        a kernel recorded a device-side fault (lola_state_check)."""
        self.check(stream)
        t = self._view_tensors(torch.device("cuda", torch.cuda.current_device()))
        view = LolaStateView(0, *[t[k].data_ptr() for k in
                                  ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v")])
        _check(self.lib.lola_state_export(self._st, ctypes.byref(view), _stream(stream)),
               "lola_state_export")
        t["n"] = int(view.n)
        return t

    def export_sequence(self, b: int, stream=None) -> Dict[str, torch.Tensor]:
        """Sequence slot b as a one-sequence state (the export layout with
        B = 1, n = its position)."""
        self.check(stream)
        t = self._view_tensors(torch.device("cuda", torch.cuda.current_device()), self.Hkv)
        view = LolaStateView(0, *[t[k].data_ptr() for k in
                                  ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v")])
        _check(self.lib.lola_state_export_sequence(self._st, int(b), ctypes.byref(view),
                                                   _stream(stream)), "lola_state_export_sequence")
        t["n"] = int(view.n)
        return t

    def import_sequence(self, b: int, st: Dict[str, torch.Tensor], stream=None):
        """Put a one-sequence state (e.g. export() of a batch-1 layer with the
        same configuration) into sequence slot b, at its own position."""
        keep = [st[k].contiguous() for k in
                ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v")]
        view = LolaStateView(int(st["n"]), *[_ptr(t).value for t in keep])
        _check(self.lib.lola_state_import_sequence(self._st, int(b), ctypes.byref(view),
                                                   _stream(stream)), "lola_state_import_sequence")

    def positions(self):
        """Position (tokens processed) of every sequence."""
        out = (ctypes.c_int64 * self.B)()
        _check(self.lib.lola_state_positions(self._st, out), "lola_state_positions")
        return [int(x) for x in out]

    def import_(self, st: Dict[str, torch.Tensor], stream=None):
        keep = [st[k].contiguous() for k in
                ("H", "s", "win_k", "win_v", "cache_pos", "cache_k", "cache_v")]
        view = LolaStateView(int(st["n"]), *[_ptr(t).value for t in keep])
        _check(self.lib.lola_state_import(self._st, ctypes.byref(view), _stream(stream)),
               "lola_state_import")
