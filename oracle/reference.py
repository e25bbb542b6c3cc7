"""GrowPage capacity-boundary oracle: Python side.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  It never imports the
HIP library or its binding, and the HIP path never imports it.

Two readings of the same steps live here:
  * the fp32 contract mode, in plain C (growpage_oracle.c, loaded with
    ctypes): the bit-exact target for every integer result (D_p, decision,
    kept set, compacted bytes);
  * the fp64 definition mode, in numpy: the textbook formulas in double
    precision, used to bound the fp32 scores (1e-3 relative) and as a sanity
    check of the fp32 contract.
Citations are to "GrowPage: On-Demand KV Budgeting for Efficient LLM
Reasoning Serving" (arXiv 2609.03494).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

GROW = 1
COMPRESS = 0
SHRINK = 2

_LIB = None


def lib():
    """Load liboracle.so, compiling it first only if it is missing."""
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        f32p = ctypes.POINTER(ctypes.c_float)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        i8p = ctypes.POINTER(ctypes.c_int8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        c_int, c_float, c_double = ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.orc_exp.argtypes = [c_float]
        L.orc_exp.restype = c_float
        L.orc_ema.argtypes = [f32p, f32p, i32p, u8p, c_int, c_int, c_int, c_int, c_int, c_float, c_float]
        L.orc_ema.restype = None
        L.orc_qhat.argtypes = [f32p, c_int, c_int, f32p, f32p, c_int, c_int, c_int, f32p]
        L.orc_qhat.restype = None
        L.orc_dp.argtypes = [f32p, c_int, c_int, c_int, c_int]
        L.orc_dp.restype = c_int
        L.orc_row.argtypes = [u16p, c_int, c_int, c_int, f32p, c_int, c_int, c_int, f32p, f32p, f32p, i32p]
        L.orc_row.restype = None
        L.orc_decide.argtypes = [i32p, i32p, c_int, ctypes.c_int64, c_double, i64p, ctypes.POINTER(c_double)]
        L.orc_decide.restype = c_int
        L.orc_grow.argtypes = [i8p, c_int, i32p, c_int, i32p, i32p, i32p, c_int, i8p, i64p]
        L.orc_grow.restype = None
        L.orc_select.argtypes = [f32p, c_int, c_int, c_int, c_int, u8p]
        L.orc_select.restype = c_int
        L.orc_select_pages.argtypes = [f32p, c_int, c_int, c_int, c_int, c_int, u8p]
        L.orc_select_pages.restype = c_int
        L.orc_decide_shrink.argtypes = [i32p, i32p, c_int, ctypes.c_int64, c_int, c_int, c_double,
                                        c_double, c_int, i64p, ctypes.POINTER(c_double)]
        L.orc_decide_shrink.restype = c_int
        L.orc_return_pages.argtypes = [i8p, c_int, i32p, c_int, i32p, i32p, i32p, i32p]
        L.orc_return_pages.restype = c_int
        L.orc_share_plan.argtypes = [i8p, c_int, i32p, c_int, i32p, i32p, i32p, i32p, i32p, u8p]
        L.orc_share_plan.restype = c_int
        L.orc_share_release.argtypes = [c_int, i32p, c_int, i32p, u8p, i32p]
        L.orc_share_release.restype = None
        L.orc_compact.argtypes = [u16p, u8p, c_int, c_int]
        L.orc_compact.restype = c_int
        _LIB = L
    return _LIB


def _p(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


@dataclass(frozen=True)
class OracleConfig:
    """Method parameters (the pages' defaults: §3.2, §3.3, §5.1, Appendix D.2)."""
    L: int
    Hq: int
    Hkv: int
    d: int = 128
    b: int = 256            # page size (§5.1)
    R: int = 16             # protected recent window (§3.3, §5.1)
    k_loc: int = 64         # local retention quota (Appendix D.2)
    p_num: int = 99         # p = 0.99 (§3.2)
    p_den: int = 100
    tau: float = 0.0        # demand threshold (§3.2, Appendix D.1)
    alpha_s: float = 0.1    # 1 - beta_S, beta_S = 0.9 (§3.2 Eq. 6)
    alpha_l: float = 0.001  # 1 - beta_L, beta_L = 0.999
    M: int = 512            # query slots (Appendix E.1)
    policy: int = 0         # 0: Grow or Compress & Hold (section 3); 1: GrowPage-Shrink (App. H.1)
    shrink_tau: float = -0.005  # Eq. 13 shrink threshold (App. H.1)
    min_tokens: int = 1024  # capacity floor of Shrink (App. H.1)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


# ---------------------------------------------------------------------------
# fp32 contract mode (C)
# ---------------------------------------------------------------------------

def exp32(x: np.ndarray) -> np.ndarray:
    L = lib()
    x = np.asarray(x, dtype=np.float32)
    return np.array([L.orc_exp(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def ema(cfg: OracleConfig, state: np.ndarray, q: np.ndarray, slot: np.ndarray,
        first_step: np.ndarray) -> None:
    """A0, in place.  state [L][M][2][Hq][d] fp32; q [B][L][Hq][d] fp32."""
    assert state.dtype == np.float32 and q.dtype == np.float32
    B = q.shape[0]
    slot = np.ascontiguousarray(slot, dtype=np.int32)
    first = np.ascontiguousarray(first_step, dtype=np.uint8)
    q = np.ascontiguousarray(q)
    lib().orc_ema(_p(state, ctypes.c_float), _p(q, ctypes.c_float), _p(slot, ctypes.c_int32),
                  _p(first, ctypes.c_uint8), B, cfg.L, state.shape[1], cfg.Hq, cfg.d,
                  np.float32(cfg.alpha_s), np.float32(cfg.alpha_l))


def qhat(cfg: OracleConfig, state: np.ndarray, slot: int, qcur: np.ndarray,
         rope_row: np.ndarray) -> np.ndarray:
    """A1 for one request: returns qhat [L][2][Hq][d] fp32."""
    out = np.empty((cfg.L, 2, cfg.Hq, cfg.d), dtype=np.float32)
    qcur = np.ascontiguousarray(qcur, dtype=np.float32)
    rope_row = np.ascontiguousarray(rope_row, dtype=np.float32)
    lib().orc_qhat(_p(state, ctypes.c_float), state.shape[1], int(slot), _p(qcur, ctypes.c_float),
                   _p(rope_row, ctypes.c_float), cfg.L, cfg.Hq, cfg.d, _p(out, ctypes.c_float))
    return out


def dp(v: np.ndarray, p_num: int = 99, p_den: int = 100) -> int:
    """D_p of one fp32 weight vector in the fp32 contract (Eq. 2)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    return int(lib().orc_dp(_p(v, ctypes.c_float), 1, v.size, p_num, p_den))


@dataclass
class RowResult:
    dp: np.ndarray          # [2] int32: K^S, K^L
    abar_all: np.ndarray    # [N][2] fp32
    abar_dem: np.ndarray    # [N-b][2] fp32
    logits: np.ndarray | None


def row(cfg: OracleConfig, keys: np.ndarray, qh: np.ndarray, want_logits: bool = False) -> RowResult:
    """A2-A4 for one (layer, KV head) row.  keys [N][d] uint16 (bf16 bits),
    qh [2][G][d] fp32."""
    keys = np.ascontiguousarray(keys, dtype=np.uint16)
    qh = np.ascontiguousarray(qh, dtype=np.float32)
    N = keys.shape[0]
    ndem = max(N - cfg.b, 0)
    G = qh.shape[1]
    aa = np.empty((N, 2), dtype=np.float32)
    ad = np.empty((max(ndem, 1), 2), dtype=np.float32)
    dpo = np.empty(2, dtype=np.int32)
    lg = np.empty((2, G, N), dtype=np.float32) if want_logits else None
    lgp = _p(lg, ctypes.c_float) if want_logits else ctypes.POINTER(ctypes.c_float)()
    lib().orc_row(_p(keys, ctypes.c_uint16), N, cfg.d, cfg.b, _p(qh, ctypes.c_float), G,
                  cfg.p_num, cfg.p_den, lgp, _p(aa, ctypes.c_float), _p(ad, ctypes.c_float),
                  _p(dpo, ctypes.c_int32))
    return RowResult(dp=dpo, abar_all=aa, abar_dem=ad[:ndem], logits=lg)


def decide(cfg: OracleConfig, ks: np.ndarray, kl: np.ndarray, card_c: int,
           num_pages: int | None = None):
    """A5 for one request: returns (decision, diff, delta).  With
    cfg.policy == 1 the three-way Shrink rule (needs num_pages)."""
    ks = np.ascontiguousarray(ks, dtype=np.int32).ravel()
    kl = np.ascontiguousarray(kl, dtype=np.int32).ravel()
    diff = ctypes.c_int64()
    delta = ctypes.c_double()
    if cfg.policy == 1:
        P = int(card_c) // cfg.b + 1 if num_pages is None else int(num_pages)
        dec = lib().orc_decide_shrink(_p(ks, ctypes.c_int32), _p(kl, ctypes.c_int32), ks.size,
                                      int(card_c), P, cfg.b, float(cfg.tau),
                                      float(cfg.shrink_tau), int(cfg.min_tokens),
                                      ctypes.byref(diff), ctypes.byref(delta))
    else:
        dec = lib().orc_decide(_p(ks, ctypes.c_int32), _p(kl, ctypes.c_int32), ks.size,
                               int(card_c), float(cfg.tau), ctypes.byref(diff),
                               ctypes.byref(delta))
    return int(dec), int(diff.value), float(delta.value)


def grow(decision: np.ndarray, block_table: np.ndarray, num_pages: np.ndarray,
         free_stack: np.ndarray, free_count: int, reserve: int = 0,
         refcount: np.ndarray | None = None):
    """A6 in place on block_table / num_pages.  Returns (action, free_count, counters).
    With reference counts (App. E.2: Grow by One Page appends a page that only
    this request references), each granted page gets a count of 1."""
    decision = np.ascontiguousarray(decision, dtype=np.int8)
    B, max_pages = block_table.shape
    assert block_table.dtype == np.int32 and num_pages.dtype == np.int32
    fc = np.array([free_count], dtype=np.int32)
    action = np.empty(B, dtype=np.int8)
    counters = np.zeros(3, dtype=np.int64)
    fs = np.ascontiguousarray(free_stack, dtype=np.int32)
    lib().orc_grow(_p(decision, ctypes.c_int8), B, _p(block_table, ctypes.c_int32), max_pages,
                   _p(num_pages, ctypes.c_int32), _p(fs, ctypes.c_int32), _p(fc, ctypes.c_int32),
                   int(reserve), _p(action, ctypes.c_int8), _p(counters, ctypes.c_int64))
    if refcount is not None:
        for r in np.nonzero(action == GROW)[0]:
            refcount[block_table[r, num_pages[r] - 1]] = 1
    return action, int(fc[0]), counters


def select(cfg: OracleConfig, abar_all: np.ndarray, k_loc: int | None = None,
           b: int | None = None, R: int | None = None, pages: int = 1) -> np.ndarray:
    """A7-A8 for one row: returns keep [N] uint8.  pages = slots freed in
    pages: 1 for Compress & Hold, 2 for Shrink."""
    abar_all = np.ascontiguousarray(abar_all, dtype=np.float32)
    N = abar_all.shape[0]
    keep = np.empty(N, dtype=np.uint8)
    rc = lib().orc_select_pages(_p(abar_all, ctypes.c_float), N, cfg.b if b is None else b,
                                cfg.R if R is None else R,
                                cfg.k_loc if k_loc is None else k_loc, int(pages),
                                _p(keep, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("local quota exceeds the retention budget")
    return keep


def return_pages(action: np.ndarray, block_table: np.ndarray, num_pages: np.ndarray,
                 free_stack: np.ndarray, free_count: int, refcount: np.ndarray | None = None):
    """Shrink's page return, in place on block_table / num_pages /
    free_stack (and refcount).  Returns (pages pushed, free_count)."""
    action = np.ascontiguousarray(action, dtype=np.int8)
    B, max_pages = block_table.shape
    assert block_table.dtype == np.int32 and num_pages.dtype == np.int32
    assert free_stack.dtype == np.int32 and free_stack.flags["C_CONTIGUOUS"]
    fc = np.array([free_count], dtype=np.int32)
    rc = ctypes.POINTER(ctypes.c_int32)()
    if refcount is not None:
        assert refcount.dtype == np.int32 and refcount.flags["C_CONTIGUOUS"]
        rc = _p(refcount, ctypes.c_int32)
    n = lib().orc_return_pages(_p(action, ctypes.c_int8), B, _p(block_table, ctypes.c_int32),
                               max_pages, _p(num_pages, ctypes.c_int32),
                               _p(free_stack, ctypes.c_int32), _p(fc, ctypes.c_int32), rc)
    return int(n), int(fc[0])


def share_plan(action: np.ndarray, block_table: np.ndarray, num_pages: np.ndarray,
               refcount: np.ndarray, free_stack: np.ndarray, free_count: int):
    """Target pages of prefix-cache-aware compression (Appendix E.2).
    Returns (target [B][max_pages], ok [B], pages allocated, free_count)."""
    action = np.ascontiguousarray(action, dtype=np.int8)
    B, max_pages = block_table.shape
    target = np.empty((B, max_pages), np.int32)
    ok = np.empty(B, np.uint8)
    fc = np.array([free_count], dtype=np.int32)
    used = lib().orc_share_plan(_p(action, ctypes.c_int8), B,
                                _p(np.ascontiguousarray(block_table, np.int32), ctypes.c_int32),
                                max_pages,
                                _p(np.ascontiguousarray(num_pages, np.int32), ctypes.c_int32),
                                _p(np.ascontiguousarray(refcount, np.int32), ctypes.c_int32),
                                _p(np.ascontiguousarray(free_stack, np.int32), ctypes.c_int32),
                                _p(fc, ctypes.c_int32), _p(target, ctypes.c_int32),
                                _p(ok, ctypes.c_uint8))
    return target, ok, int(used), int(fc[0])


def share_release(block_table: np.ndarray, target: np.ndarray, ok: np.ndarray,
                  refcount: np.ndarray) -> None:
    """Swap replaced pages for their targets and move the references, in place."""
    B, max_pages = block_table.shape
    assert block_table.dtype == np.int32 and refcount.dtype == np.int32
    lib().orc_share_release(B, _p(block_table, ctypes.c_int32), max_pages,
                            _p(np.ascontiguousarray(target, np.int32), ctypes.c_int32),
                            _p(np.ascontiguousarray(ok, np.uint8), ctypes.c_uint8),
                            _p(refcount, ctypes.c_int32))


def compact(rows: np.ndarray, keep: np.ndarray) -> int:
    """A9 in place on one row chain rows [N][width] (16-bit elements)."""
    assert rows.dtype == np.uint16 and rows.flags["C_CONTIGUOUS"]
    keep = np.ascontiguousarray(keep, dtype=np.uint8)
    return int(lib().orc_compact(_p(rows, ctypes.c_uint16), _p(keep, ctypes.c_uint8),
                                 rows.shape[0], int(np.prod(rows.shape[1:]))))


# ---------------------------------------------------------------------------
# Event orchestration over a paged pool (numpy copies of the touched pages)
# ---------------------------------------------------------------------------

def gather_row(k_pool: np.ndarray, layer: int, head: int, pages) -> np.ndarray:
    """Logical slot order of one row from a pool laid out
    [L][pool_pages][Hkv][b][d]: slot i lives in pages[i // b] at i % b."""
    t = k_pool[layer, np.asarray(pages, dtype=np.int64), head]  # [P][b][d]
    return np.ascontiguousarray(t.reshape(-1, t.shape[-1]))


def demand(cfg: OracleConfig, get_keys, block_table, num_pages, state, qcur, rope,
           positions, slots, want_abar: bool = False):
    """A1-A5 for a batch.  get_keys(r, layer, head, pages) -> [N][d] uint16.
    qcur [B][L][Hq][d]; rope [max_pos][d].  Returns a dict."""
    B = len(num_pages)
    G = cfg.G
    ks = np.zeros((B, cfg.L, cfg.Hkv), dtype=np.int32)
    kl = np.zeros((B, cfg.L, cfg.Hkv), dtype=np.int32)
    decision = np.zeros(B, dtype=np.int8)
    diff = np.zeros(B, dtype=np.int64)
    delta = np.zeros(B, dtype=np.float64)
    abar = {}
    for r in range(B):
        P = int(num_pages[r])
        pages = block_table[r, :P]
        qh = qhat(cfg, state, int(slots[r]), qcur[r], rope[int(positions[r])])
        for l in range(cfg.L):
            for h in range(cfg.Hkv):
                keys = get_keys(r, l, h, pages)
                q2 = np.ascontiguousarray(qh[l][:, h * G:(h + 1) * G])
                res = row(cfg, keys, q2)
                ks[r, l, h], kl[r, l, h] = res.dp
                if want_abar:
                    abar[(r, l, h)] = res.abar_all
        decision[r], diff[r], delta[r] = decide(cfg, ks[r], kl[r], (P - 1) * cfg.b, P)
    return dict(ks=ks, kl=kl, decision=decision, diff=diff, delta=delta, abar=abar)


# ---------------------------------------------------------------------------
# fp64 definition mode (numpy)
# ---------------------------------------------------------------------------

def bf16_to_f64(keys: np.ndarray) -> np.ndarray:
    return (keys.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ema_f64(qs: np.ndarray, alpha: float) -> np.ndarray:
    """Eq. 6 in fp64 over a stream qs [T][...] with the first-step init."""
    s = qs[0].astype(np.float64)
    beta = 1.0 - alpha
    for t in range(1, qs.shape[0]):
        s = beta * s + (1.0 - beta) * qs[t].astype(np.float64)
    return s


def qhat_f64(qbar: np.ndarray, qt: np.ndarray, rope_row: np.ndarray) -> np.ndarray:
    """Eq. 12 then rotary embedding then 1/sqrt(d), fp64.  qbar [..][d]."""
    qbar = qbar.astype(np.float64)
    qt = qt.astype(np.float64)
    d = qbar.shape[-1]
    h = d // 2
    rms_q = np.sqrt(np.mean(qt * qt, axis=-1, keepdims=True))
    rms_b = np.sqrt(np.mean(qbar * qbar, axis=-1, keepdims=True))
    gamma = np.where(rms_b > 0, rms_q / np.where(rms_b > 0, rms_b, 1.0), 0.0)
    x = gamma * qbar
    c = rope_row[:h].astype(np.float64)
    s = rope_row[h:].astype(np.float64)
    y = np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], axis=-1)
    return y / np.sqrt(d)


def softmax_f64(l: np.ndarray) -> np.ndarray:
    m = np.max(l, axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def dp_f64(a: np.ndarray, p: float) -> int:
    """Eq. 2 in fp64: sort descending, prefix-sum, first k reaching p * total."""
    a = np.sort(np.asarray(a, dtype=np.float64))[::-1]
    c = np.cumsum(a)
    k = int(np.searchsorted(c, p * c[-1] * (1 - 1e-15), side="left")) + 1
    return min(k, a.size)


def row_f64(keys_f64: np.ndarray, qh_f64: np.ndarray, b: int, p: float = 0.99):
    """A2-A4 in fp64 for one row.  keys [N][d], qh [2][G][d]."""
    N = keys_f64.shape[0]
    ndem = N - b
    lg = qh_f64 @ keys_f64.T  # [2][G][N]
    a_all = softmax_f64(lg).mean(axis=1)  # [2][N]
    a_dem = softmax_f64(lg[..., :ndem]).mean(axis=1) if ndem > 0 else np.zeros((2, 0))
    dps = [dp_f64(a_dem[x], p) if ndem > 0 else 0 for x in range(2)]
    return dict(abar_all=a_all.T.copy(), abar_dem=a_dem.T.copy(), dp=np.array(dps), logits=lg)


# ---------------------------------------------------------------------------
# Decode step (fp64 definition mode): the regular decoding path whose
# attention kernel also carries the summary update (§4.1 "Lightweight
# Per-Request State Management"; App. E.1 "Initialization and online
# update"), and the retained-subset output of §3.1 Eq. 3 and Eq. 5.
# ---------------------------------------------------------------------------

def rope_f64(x: np.ndarray, rope_row: np.ndarray) -> np.ndarray:
    """Rotary embedding at one position, pairs (j, j + d/2): the same
    rotate-half convention the cached keys were stored with.  x [..][d]."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    c = rope_row[:h].astype(np.float64)
    s = rope_row[h:].astype(np.float64)
    return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s],
                          axis=-1)


def decode_attention_f64(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                         rope_row: np.ndarray):
    """Full-cache attention output o_t of §3.1 Eq. 3 for the G query heads
    of one KV head at one decode step.  q [G][d] (normalised, pre-RoPE),
    keys / values [N][d] bf16 bits (keys post-RoPE at their own positions).
    The query is rotated to its position and scaled by 1/sqrt(d); each head
    takes a softmax over the N slots.  Returns (o [G][d], a [G][N])."""
    d = q.shape[-1]
    qh = rope_f64(q, rope_row) / np.sqrt(d)
    a = softmax_f64(qh @ bf16_to_f64(keys).T)
    return a @ bf16_to_f64(values), a


def subset_output_f64(a: np.ndarray, values: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """Retained-subset output of §3.1 Eq. 3: weights a on the slots of keep,
    renormalised by their mass m(S).  a [G][N], values [N][d] bf16 bits,
    keep [N] bool."""
    keep = np.asarray(keep, dtype=bool)
    m = a[:, keep].sum(axis=1, keepdims=True)
    return (a[:, keep] / m) @ bf16_to_f64(values)[keep]


def worst_case_error_f64(a: np.ndarray, keep: np.ndarray, v_max: float) -> np.ndarray:
    """§3.1 Eq. 5: sup over values of norm at most v_max of the output error
    of retaining keep, = 2 v_max (1 - m(S)), per head.  a [G][N]."""
    keep = np.asarray(keep, dtype=bool)
    return 2.0 * v_max * (1.0 - a[:, keep].sum(axis=1))
