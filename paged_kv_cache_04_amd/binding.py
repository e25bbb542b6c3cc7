"""Thin Python binding of libgrowpage.so (include/growpage.h).

Argument marshalling only: every step of the boundary event runs in the HIP
kernels behind the C ABI.  Tensors are torch device tensors; the binding
passes their data pointers and the current HIP stream.  If the library is not
built, importing works but every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgrowpage.so")

GP_COMPRESS = 0
GP_GROW = 1
GP_SHRINK = 2
GP_POLICY_GROWPAGE = 0
GP_POLICY_SHRINK = 1

SYMBOLS = (
    "gp_create", "gp_destroy", "gp_workspace_bytes", "gp_update_summaries", "gp_demand",
    "gp_grow_page", "gp_compress_hold", "gp_get_counters", "gp_get_device_errors",
    "gp_status_str", "gp_last_hip_error", "gp_profile", "gp_profile_read",
    "gp_decode_workspace_bytes", "gp_decode_attention", "gp_decode_attention_static",
)

# bytes of the library's per-GPU scratch buffer (gp_decode_attention_static)
GP_STATIC_SCRATCH_BYTES = 64 << 20

# bandwidth probes (include/gp_probe.h)
PROBE_SYMBOLS = ("gp_probe_read", "gp_probe_copy")
GP_PROBE_BLOCK_BYTES = 16384

KERNELS = ("ema", "plan", "qhat", "demand", "decide", "grow", "select", "compact", "return",
           "share", "decode")


class GPError(RuntimeError):
    pass


class gp_config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("recent_window", ctypes.c_int32),
        ("local_quota", ctypes.c_int32), ("p_num", ctypes.c_int32), ("p_den", ctypes.c_int32),
        ("tau", ctypes.c_double), ("alpha_short", ctypes.c_float),
        ("alpha_long", ctypes.c_float), ("max_slots", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("shrink_tau", ctypes.c_double),
        ("min_tokens", ctypes.c_int32), ("compact_workgroups", ctypes.c_int32),
    ]


class gp_pool(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
        ("free_stack", ctypes.c_void_p), ("free_count", ctypes.c_void_p),
        ("refcount", ctypes.c_void_p),
    ]


class gp_batch(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("block_table", ctypes.c_void_p), ("num_pages", ctypes.c_void_p),
        ("num_tokens", ctypes.c_void_p), ("slot", ctypes.c_void_p),
        ("position", ctypes.c_void_p), ("num_pages_host", ctypes.c_void_p),
    ]


class gp_demand_out(ctypes.Structure):
    _fields_ = [
        ("k_short", ctypes.c_void_p), ("k_long", ctypes.c_void_p), ("k_diff", ctypes.c_void_p),
        ("delta", ctypes.c_void_p), ("decision", ctypes.c_void_p), ("abar", ctypes.c_void_p),
    ]


class gp_kernel_times(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(KERNELS)), ("launches", ctypes.c_int64 * len(KERNELS))]


class gp_counters(ctypes.Structure):
    _fields_ = [("grown", ctypes.c_int64), ("compress", ctypes.c_int64),
                ("fallback", ctypes.c_int64), ("shrunk", ctypes.c_int64),
                ("copied", ctypes.c_int64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libgrowpage.so; raises if it is missing (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise GPError(f"{path} is not built: run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.gp_create.argtypes = [ctypes.POINTER(gp_config), ctypes.POINTER(vp)]
    L.gp_create.restype = ctypes.c_int
    L.gp_destroy.argtypes = [vp]
    L.gp_destroy.restype = None
    L.gp_workspace_bytes.argtypes = [vp, i32, i64, i64]
    L.gp_workspace_bytes.restype = sz
    L.gp_update_summaries.argtypes = [vp, vp, vp, vp, vp, i32, vp]
    L.gp_update_summaries.restype = ctypes.c_int
    L.gp_demand.argtypes = [vp, ctypes.POINTER(gp_pool), ctypes.POINTER(gp_batch), vp, vp, vp,
                            i32, vp, sz, ctypes.POINTER(gp_demand_out), vp]
    L.gp_demand.restype = ctypes.c_int
    L.gp_grow_page.argtypes = [vp, ctypes.POINTER(gp_pool), ctypes.POINTER(gp_batch), vp, vp,
                               i32, vp]
    L.gp_grow_page.restype = ctypes.c_int
    L.gp_compress_hold.argtypes = [vp, ctypes.POINTER(gp_pool), ctypes.POINTER(gp_batch), vp,
                                   vp, sz, vp, vp]
    L.gp_compress_hold.restype = ctypes.c_int
    L.gp_decode_workspace_bytes.argtypes = [vp, i32, i64]
    L.gp_decode_workspace_bytes.restype = sz
    L.gp_decode_attention.argtypes = [vp, ctypes.POINTER(gp_pool), ctypes.POINTER(gp_batch), i32,
                                      vp, vp, vp, vp, i32, vp, vp, sz, vp]
    L.gp_decode_attention.restype = ctypes.c_int
    L.gp_decode_attention_static.argtypes = [vp, ctypes.POINTER(gp_pool),
                                             ctypes.POINTER(gp_batch), i32, vp, vp, vp, vp,
                                             i32, vp, vp]
    L.gp_decode_attention_static.restype = ctypes.c_int
    L.gp_probe_read.argtypes = [vp, sz, vp, vp]
    L.gp_probe_read.restype = ctypes.c_int
    L.gp_probe_copy.argtypes = [vp, vp, sz, vp]
    L.gp_probe_copy.restype = ctypes.c_int
    L.gp_get_counters.argtypes = [vp, ctypes.POINTER(gp_counters)]
    L.gp_get_counters.restype = ctypes.c_int
    L.gp_get_device_errors.argtypes = [vp, ctypes.POINTER(i32)]
    L.gp_get_device_errors.restype = ctypes.c_int
    L.gp_status_str.argtypes = [ctypes.c_int]
    L.gp_status_str.restype = ctypes.c_char_p
    L.gp_last_hip_error.argtypes = [vp]
    L.gp_last_hip_error.restype = ctypes.c_int
    L.gp_profile.argtypes = [vp, ctypes.c_int]
    L.gp_profile.restype = ctypes.c_int
    L.gp_profile_read.argtypes = [vp, ctypes.POINTER(gp_kernel_times)]
    L.gp_profile_read.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int, what: str, ctx=None):
    if status != 0:
        msg = load().gp_status_str(status).decode()
        hip = load().gp_last_hip_error(ctx.handle) if ctx is not None else 0
        raise GPError(f"{what}: {msg} (status {status}, hip error {hip})")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.is_contiguous(), "tensors passed to the library must be contiguous"
        return t.data_ptr()
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    raise TypeError(type(t))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class Config:
    """Method parameters; defaults are the pages' (see include/growpage.h)."""
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = 128
    page_size: int = 256
    recent_window: int = 16
    local_quota: int = 64
    p_num: int = 99
    p_den: int = 100
    tau: float = 0.0
    alpha_short: float = 0.1
    alpha_long: float = 0.001
    max_slots: int = 512
    policy: int = GP_POLICY_GROWPAGE
    shrink_tau: float = -0.005
    min_tokens: int = 1024
    compact_workgroups: int = 0  # 0: 2 per CU

    @property
    def max_freed(self) -> int:
        """Pages of slots one event can free per request (2 with Shrink)."""
        return 2 if self.policy == GP_POLICY_SHRINK else 1


class Context:
    """Owns a gp_ctx (created on the current device)."""

    def __init__(self, cfg: Config):
        L = load()
        self.cfg = cfg
        c = gp_config(cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim,
                      cfg.page_size, cfg.recent_window, cfg.local_quota, cfg.p_num, cfg.p_den,
                      float(cfg.tau), float(cfg.alpha_short), float(cfg.alpha_long),
                      cfg.max_slots, cfg.policy, float(cfg.shrink_tau), cfg.min_tokens,
                      cfg.compact_workgroups)
        h = ctypes.c_void_p()
        _check(L.gp_create(ctypes.byref(c), ctypes.byref(h)), "gp_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            load().gp_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass
class Pool:
    k_pool: torch.Tensor      # bf16 [L][num_pages][Hkv][b][d]
    v_pool: torch.Tensor
    free_stack: torch.Tensor  # int32 [num_pages]
    free_count: torch.Tensor  # int32 [1]
    refcount: torch.Tensor | None = None  # int32 [num_pages], prefix sharing

    def c(self) -> gp_pool:
        return gp_pool(_ptr(self.k_pool), _ptr(self.v_pool), int(self.k_pool.shape[1]),
                       _ptr(self.free_stack), _ptr(self.free_count), _ptr(self.refcount))


@dataclass
class Batch:
    block_table: torch.Tensor     # int32 [B][max_pages]
    num_pages: torch.Tensor       # int32 [B]
    num_tokens: torch.Tensor      # int32 [B]
    slot: torch.Tensor            # int32 [B]
    position: torch.Tensor        # int32 [B]
    num_pages_host: np.ndarray    # int32 [B] (host mirror)

    def c(self) -> gp_batch:
        return gp_batch(int(self.block_table.shape[0]), int(self.block_table.shape[1]),
                        _ptr(self.block_table), _ptr(self.num_pages), _ptr(self.num_tokens),
                        _ptr(self.slot), _ptr(self.position), _ptr(self.num_pages_host))


@dataclass
class DemandOut:
    k_short: torch.Tensor   # int32 [B][L][Hkv]
    k_long: torch.Tensor
    k_diff: torch.Tensor    # int64 [B]
    delta: torch.Tensor     # float64 [B]
    decision: torch.Tensor  # int8 [B]
    abar: torch.Tensor | None = None  # fp32 [sum of row tokens][2]

    @staticmethod
    def empty(cfg: Config, B: int, device, abar_tokens: int | None = None) -> "DemandOut":
        i32 = dict(dtype=torch.int32, device=device)
        return DemandOut(
            torch.empty((B, cfg.num_layers, cfg.num_kv_heads), **i32),
            torch.empty((B, cfg.num_layers, cfg.num_kv_heads), **i32),
            torch.empty(B, dtype=torch.int64, device=device),
            torch.empty(B, dtype=torch.float64, device=device),
            torch.empty(B, dtype=torch.int8, device=device),
            None if abar_tokens is None else torch.empty((abar_tokens, 2), dtype=torch.float32,
                                                         device=device))

    def c(self) -> gp_demand_out:
        return gp_demand_out(_ptr(self.k_short), _ptr(self.k_long), _ptr(self.k_diff),
                             _ptr(self.delta), _ptr(self.decision), _ptr(self.abar))


def gp_workspace_bytes(ctx: Context, batch: int, total_tokens: int, max_tokens: int) -> int:
    return int(load().gp_workspace_bytes(ctx.handle, batch, total_tokens, max_tokens))


def gp_update_summaries(ctx: Context, qstate, q, slot, first_step, stream=None):
    _check(load().gp_update_summaries(ctx.handle, _ptr(qstate), _ptr(q), _ptr(slot),
                                      _ptr(first_step), int(q.shape[0]), _stream(stream)),
           "gp_update_summaries", ctx)


def gp_demand(ctx: Context, pool: Pool, batch: Batch, qstate, q_cur, rope, workspace,
              out: DemandOut, stream=None):
    p, b, o = pool.c(), batch.c(), out.c()
    _check(load().gp_demand(ctx.handle, ctypes.byref(p), ctypes.byref(b), _ptr(qstate),
                            _ptr(q_cur), _ptr(rope), int(rope.shape[0]), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), ctypes.byref(o),
                            _stream(stream)), "gp_demand", ctx)


def gp_grow_page(ctx: Context, pool: Pool, batch: Batch, decision, action, reserve_pages: int = 0,
                 stream=None):
    p, b = pool.c(), batch.c()
    _check(load().gp_grow_page(ctx.handle, ctypes.byref(p), ctypes.byref(b), _ptr(decision),
                               _ptr(action), int(reserve_pages), _stream(stream)),
           "gp_grow_page", ctx)


def gp_compress_hold(ctx: Context, pool: Pool, batch: Batch, action, workspace,
                     dropped_out=None, stream=None):
    p, b = pool.c(), batch.c()
    _check(load().gp_compress_hold(ctx.handle, ctypes.byref(p), ctypes.byref(b), _ptr(action),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _ptr(dropped_out), _stream(stream)), "gp_compress_hold", ctx)


def gp_decode_workspace_bytes(ctx: Context, batch: int, total_pages: int) -> int:
    return int(load().gp_decode_workspace_bytes(ctx.handle, batch, total_pages))


def gp_decode_attention(ctx: Context, pool: Pool, batch: Batch, layer: int, q, qstate, first_step,
                        rope, out, workspace, stream=None):
    p, b = pool.c(), batch.c()
    _check(load().gp_decode_attention(ctx.handle, ctypes.byref(p), ctypes.byref(b), int(layer),
                                      _ptr(q), _ptr(qstate), _ptr(first_step), _ptr(rope),
                                      int(rope.shape[0]), _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "gp_decode_attention", ctx)


def gp_decode_attention_static(ctx: Context, pool: Pool, batch: Batch, layer: int, q, qstate,
                               first_step, rope, out, stream=None):
    """gp_decode_attention with the scratch in the library's per-GPU buffer
    (no workspace argument; allocates nothing)."""
    p, b = pool.c(), batch.c()
    _check(load().gp_decode_attention_static(ctx.handle, ctypes.byref(p), ctypes.byref(b),
                                             int(layer), _ptr(q), _ptr(qstate), _ptr(first_step),
                                             _ptr(rope), int(rope.shape[0]), _ptr(out),
                                             _stream(stream)), "gp_decode_attention_static", ctx)


def gp_probe_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Streaming read of every byte of src (include/gp_probe.h)."""
    rc = load().gp_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                              _stream(stream))
    if rc != 0:
        raise GPError(f"gp_probe_read: HIP error {rc}")


def gp_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Streaming copy of src into dst (include/gp_probe.h)."""
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    rc = load().gp_probe_copy(_ptr(src), _ptr(dst), n, _stream(stream))
    if rc != 0:
        raise GPError(f"gp_probe_copy: HIP error {rc}")


def gp_get_counters(ctx: Context) -> dict:
    c = gp_counters()
    _check(load().gp_get_counters(ctx.handle, ctypes.byref(c)), "gp_get_counters", ctx)
    return dict(grown=c.grown, compress=c.compress, fallback=c.fallback, shrunk=c.shrunk,
                copied=c.copied)


def gp_get_device_errors(ctx: Context) -> int:
    v = ctypes.c_int32()
    _check(load().gp_get_device_errors(ctx.handle, ctypes.byref(v)), "gp_get_device_errors", ctx)
    return int(v.value)


def gp_profile(ctx: Context, enable: bool):
    _check(load().gp_profile(ctx.handle, 1 if enable else 0), "gp_profile", ctx)


def gp_profile_read(ctx: Context) -> dict:
    """{kernel name: (total ms, launches)} accumulated since gp_profile(ctx, True)."""
    t = gp_kernel_times()
    _check(load().gp_profile_read(ctx.handle, ctypes.byref(t)), "gp_profile_read", ctx)
    return {k: (float(t.ms[i]), int(t.launches[i])) for i, k in enumerate(KERNELS)}
