"""Thin ctypes binding of libprsink.so (the PR-Sink C ABI in include/pr_sink.h).

Argument marshalling only: tensors become device pointers, the stream is
torch's current stream on the tensors' device.  Every step of the path runs
in the library's HIP kernels; there is no fallback.  If the library is not
built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_double, c_int32, c_size_t, c_void_p

import numpy as np

from .build import LIB_PATH
from .synth import DTYPE_BF16, PRSinkConfig

PR_SINK_OK, PR_SINK_EINVAL, PR_SINK_ESTATE, PR_SINK_ENOSPACE, PR_SINK_EHIP = 0, -1, -2, -3, -4
SLOT_REF, SLOT_STATIC, SLOT_DYNAMIC, SLOT_WINDOW0 = 0, 1, 2, 3

EXPORTED = (
    "pr_sink_arena_bytes", "pr_sink_cache_init", "pr_sink_set_ref", "pr_sink_retrieve",
    "pr_sink_attend", "pr_sink_clean_kv_write", "pr_sink_bank_update", "pr_sink_bank_state",
    "pr_sink_slot_view", "pr_sink_segments", "pr_sink_set_attend_events", "pr_sink_cache_destroy",
    "pr_sink_last_error", "pr_sink_attend_noalloc",
)


class CConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("n_heads", c_int32), ("head_dim", c_int32),
        ("rope_dims", c_int32 * 3), ("rope_theta", c_double),
        ("lat_h", c_int32), ("lat_w", c_int32), ("ref_frames", c_int32),
        ("block_frames", c_int32), ("window_slots", c_int32), ("bank_size", c_int32),
        ("bank_fill_blocks", c_int32), ("fp_dim", c_int32), ("dtype", c_int32), ("t0", c_int32),
        ("bank_policy", c_int32), ("bank_stale_blocks", c_int32), ("bank_refresh_tau", c_double),
    ]


def to_c_config(cfg: PRSinkConfig) -> CConfig:
    return CConfig(cfg.n_layers, cfg.n_heads, cfg.head_dim, (c_int32 * 3)(*cfg.rope_dims),
                   float(cfg.rope_theta), cfg.lat_h, cfg.lat_w, cfg.ref_frames, cfg.block_frames,
                   cfg.window_slots, cfg.bank_size, cfg.bank_fill_blocks, cfg.fp_dim,
                   0 if cfg.dtype == DTYPE_BF16 else 1, cfg.t0, cfg.bank_policy,
                   cfg.bank_stale_blocks, float(cfg.bank_refresh_tau))


class PRSinkError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pr_sink error {code}: {msg}")
        self.code = code


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, pcfg = c_void_p, c_int32, POINTER(CConfig)
        sig = {
            "pr_sink_arena_bytes": (c_size_t, [pcfg]),
            "pr_sink_cache_init": (i32, [pcfg, vp, c_size_t, vp, POINTER(vp)]),
            "pr_sink_set_ref": (i32, [vp, i32, vp, vp, vp]),
            "pr_sink_retrieve": (i32, [vp, i32, vp, vp, vp]),
            "pr_sink_attend": (i32, [vp, i32, vp, vp, vp, vp, vp]),
            "pr_sink_attend_noalloc": (i32, [vp, i32, vp, vp, vp, vp, vp]),
            "pr_sink_clean_kv_write": (i32, [vp, i32, vp, vp, vp]),
            "pr_sink_bank_update": (i32, [vp, i32, vp]),
            "pr_sink_bank_state": (i32, [vp, vp, vp, vp, vp]),
            "pr_sink_slot_view": (i32, [vp, i32, i32, POINTER(vp), POINTER(vp), POINTER(vp),
                                        POINTER(i32)]),
            "pr_sink_segments": (i32, [vp, vp, vp, POINTER(i32)]),
            "pr_sink_set_attend_events": (i32, [vp, vp, vp]),
            "pr_sink_cache_destroy": (i32, [vp]),
            "pr_sink_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().pr_sink_last_error().decode()


def check(code: int) -> None:
    if code != PR_SINK_OK:
        raise PRSinkError(code, last_error())


def arena_bytes(cfg: PRSinkConfig) -> int:
    c = to_c_config(cfg)
    n = lib().pr_sink_arena_bytes(byref(c))
    if n == 0:
        raise PRSinkError(PR_SINK_EINVAL, last_error())
    return n


def _torch():
    import torch
    return torch


class PRSinkCache:
    """One bounded PR-Sink cache over a torch-allocated device arena.

    dry_run=True builds the host-side state machine only (no device, no
    arena): argument and call-order validation without a GPU.
    """

    def __init__(self, cfg: PRSinkConfig, device=None, arena=None, dry_run: bool = False):
        self.cfg = cfg
        self._c = to_c_config(cfg)
        self.nbytes = arena_bytes(cfg)
        self.dry_run = dry_run
        self._h = c_void_p()
        self._attend_events = None  # kept alive while the library records them
        if dry_run:
            self.arena = None
            check(lib().pr_sink_cache_init(byref(self._c), None, 0, None, byref(self._h)))
            self.device = None
            return
        torch = _torch()
        if arena is None:
            arena = torch.empty(self.nbytes, dtype=torch.uint8, device=device or "cuda")
        if arena.dtype != torch.uint8 or not arena.is_cuda or arena.numel() < self.nbytes:
            raise ValueError("arena must be a CUDA uint8 tensor of at least arena_bytes(cfg)")
        self.arena = arena
        self.device = arena.device
        check(lib().pr_sink_cache_init(byref(self._c), arena.data_ptr(), arena.numel(),
                                       self._stream(), byref(self._h)))

    # -- plumbing ------------------------------------------------------------
    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.cfg.dtype == DTYPE_BF16 else torch.float32

    def _stream(self):
        if self.dry_run:
            return None
        return c_void_p(_torch().cuda.current_stream(self.device).cuda_stream)

    def _ptr(self, t, n_tokens=None, name="tensor"):
        if self.dry_run:
            return t  # fake pointers are fine: nothing is dereferenced
        if not t.is_cuda or t.device != self.device:
            raise ValueError(f"{name} must live on {self.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if n_tokens is not None:
            shape = (n_tokens, self.cfg.n_heads, self.cfg.head_dim)
            if tuple(t.shape) != shape or t.dtype != self.torch_dtype:
                raise ValueError(f"{name} must be {self.torch_dtype} of shape {shape}, "
                                 f"got {t.dtype} {tuple(t.shape)}")
        return t.data_ptr()

    # -- the calls of the C ABI ----------------------------------------------
    def set_ref(self, layer: int, k, v):
        n = self.cfg.ref_tokens
        check(lib().pr_sink_set_ref(self._h, layer, self._ptr(k, n, "k"), self._ptr(v, n, "v"),
                                    self._stream()))

    def retrieve(self, block: int, fp_raw, slot_out=None):
        if not self.dry_run:
            torch = _torch()
            if fp_raw.dtype != torch.float32 or fp_raw.numel() != self.cfg.fp_dim:
                raise ValueError("fp_raw must be float32[fp_dim]")
            if slot_out is not None and (slot_out.dtype != torch.int32 or slot_out.numel() < 1):
                raise ValueError("slot_out must be int32 with at least one element")
        so = None if slot_out is None else self._ptr(slot_out, None, "slot_out")
        check(lib().pr_sink_retrieve(self._h, block, self._ptr(fp_raw, None, "fp_raw"), so,
                                     self._stream()))

    def attend(self, layer: int, q, k, v, out=None):
        n = self.cfg.block_tokens
        if out is None and not self.dry_run:
            out = _torch().empty_like(q)
        check(lib().pr_sink_attend(self._h, layer, self._ptr(q, n, "q"), self._ptr(k, n, "k"),
                                   self._ptr(v, n, "v"), self._ptr(out, n, "out"),
                                   self._stream()))
        return out

    def attend_noalloc(self, layer: int, q, k, v, out):
        """pr_sink_attend_noalloc: the same attention call with its scratch in the
        library's static device array (calls on one GPU must not overlap); the
        caller passes the output tensor, nothing is allocated."""
        n = self.cfg.block_tokens
        check(lib().pr_sink_attend_noalloc(self._h, layer, self._ptr(q, n, "q"), self._ptr(k, n, "k"),
                                           self._ptr(v, n, "v"), self._ptr(out, n, "out"),
                                           self._stream()))
        return out

    def clean_kv_write(self, layer: int, k, v):
        n = self.cfg.block_tokens
        check(lib().pr_sink_clean_kv_write(self._h, layer, self._ptr(k, n, "k"),
                                           self._ptr(v, n, "v"), self._stream()))

    def bank_update(self, block: int):
        check(lib().pr_sink_bank_update(self._h, block, self._stream()))

    def bank_state(self):
        """(ids int32[M], phi float64[M][fp_dim], (last_r, dyn_id, decision)); synchronises."""
        m, f = self.cfg.bank_size, self.cfg.fp_dim
        ids = np.zeros(m, np.int32)
        phi = np.zeros((m, f), np.float64)
        misc = np.zeros(3, np.int32)
        check(lib().pr_sink_bank_state(self._h, ids.ctypes.data, phi.ctypes.data,
                                       misc.ctypes.data, self._stream()))
        return ids, phi, tuple(int(x) for x in misc)

    def set_attend_events(self, start=None, stop=None):
        """Records torch.cuda.Events (timing enabled, already created, i.e.
        recorded once) around every later attention kernel; no arguments turns
        it off.  The cache keeps the two events alive while they are in use."""
        if (start is None) != (stop is None):
            raise ValueError("set both events or neither")
        if start is not None:
            for e in (start, stop):
                if not e.cuda_event:
                    raise ValueError("event has no HIP event yet: record it once before handing it over")
            check(lib().pr_sink_set_attend_events(self._h, c_void_p(start.cuda_event),
                                                  c_void_p(stop.cuda_event)))
            self._attend_events = (start, stop)
        else:
            check(lib().pr_sink_set_attend_events(self._h, None, None))
            self._attend_events = None

    def segments(self):
        """[(tokens, t_start)] of the open block in cache order."""
        tok = np.zeros(8, np.int32)
        ts = np.zeros(8, np.int32)
        n = c_int32()
        check(lib().pr_sink_segments(self._h, tok.ctypes.data, ts.ctypes.data, byref(n)))
        return [(int(tok[i]), int(ts[i])) for i in range(n.value)]

    def slot_view(self, slot: int, layer: int, rotated: bool = False):
        """Torch views of one slot's raw K and V, [t_pad][H][d] each; with
        rotated=True also its rotated K.  The raw K is None where the cache
        keeps none (the Static Sink and bank entries)."""
        k, v, r, tp = c_void_p(), c_void_p(), c_void_p(), c_int32()
        check(lib().pr_sink_slot_view(self._h, slot, layer, byref(k), byref(v), byref(r), byref(tp)))
        c = self.cfg
        n = c.n_heads * tp.value * c.head_dim
        esz = 2 if c.dtype == DTYPE_BF16 else 4
        base = self.arena.data_ptr()

        def view(ptr):
            if not ptr:
                return None
            t = self.arena[ptr - base:ptr - base + n * esz].view(self.torch_dtype)
            return t.view(tp.value, c.n_heads, c.head_dim)

        if rotated:
            return view(k.value), view(v.value), view(r.value)
        return view(k.value), view(v.value)

    def slot_index_bank(self, i: int) -> int:
        return SLOT_WINDOW0 + self.cfg.window_slots + i

    def close(self):
        if self._h:
            lib().pr_sink_cache_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
