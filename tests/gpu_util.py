"""Helpers shared by the GPU parity tests: wiring a synthetic workload into
the binding, and running the oracle on host copies of the same inputs."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import OracleConfig
from paged_kv_cache_04_amd import binding as gb
from paged_kv_cache_04_amd.runner import BoundaryRunner


def log(msg: str):
    print(msg, flush=True)


def gb_config(shape, **kw) -> gb.Config:
    return gb.Config(num_layers=shape.L, num_q_heads=shape.Hq, num_kv_heads=shape.Hkv,
                     head_dim=shape.d, page_size=shape.b, **kw)


def oracle_config(cfg: gb.Config) -> OracleConfig:
    return OracleConfig(L=cfg.num_layers, Hq=cfg.num_q_heads, Hkv=cfg.num_kv_heads,
                        d=cfg.head_dim, b=cfg.page_size, R=cfg.recent_window,
                        k_loc=cfg.local_quota, p_num=cfg.p_num, p_den=cfg.p_den, tau=cfg.tau,
                        alpha_s=cfg.alpha_short, alpha_l=cfg.alpha_long, M=cfg.max_slots,
                        policy=cfg.policy, shrink_tau=cfg.shrink_tau, min_tokens=cfg.min_tokens)


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def runner_for(wl, cfg: gb.Config, want_abar=True, want_dropped=True,
               qstate: torch.Tensor | None = None,
               refcount: torch.Tensor | None = None) -> BoundaryRunner:
    """A runner over the workload's current batch state (page counts read
    back from the device); qstate is reused when given; refcount (int32 per
    pool page) turns on prefix-preserving compression."""
    s = wl.shape
    if qstate is None:
        qstate = torch.zeros((s.L, wl.max_slots, 2, s.Hq, s.d), dtype=torch.float32,
                             device=wl.device)
    pool = gb.Pool(wl.k_pool, wl.v_pool, wl.free_stack, wl.free_count, refcount)
    batch = gb.Batch(wl.block_table, wl.num_pages, wl.num_tokens, wl.slot, wl.position,
                     wl.num_pages.cpu().numpy().astype(np.int32).copy())
    return BoundaryRunner(cfg, pool, batch, qstate, wl.rope, want_abar=want_abar,
                          want_dropped=want_dropped)


def run_stream_gpu(run: BoundaryRunner, wl, steps=None):
    steps = wl.steps if steps is None else steps
    q = None
    for t in range(steps):
        q = wl.query(t)
        run.update(q, wl.first_step(t))
    return q


def run_stream_oracle(wl, ocfg: OracleConfig, state=None, steps=None):
    steps = wl.steps if steps is None else steps
    if state is None:
        state = np.zeros((ocfg.L, wl.max_slots, 2, ocfg.Hq, ocfg.d), dtype=np.float32)
    slot = wl.slot.cpu().numpy()
    q = None
    for t in range(steps):
        q = wl.query(t).cpu().numpy()
        oracle.ema(ocfg, state, q, slot, wl.first_step(t).cpu().numpy())
    return state, q


class HostCopy:
    """Host copies of the inputs the oracle needs: only the pages the batch's
    block tables reference are copied (pools of the full-size workloads are
    far larger than host memory), with a map from pool page ids to them."""

    def __init__(self, wl):
        self.bt = wl.block_table.cpu().numpy().copy()
        self.P = wl.num_pages.cpu().numpy().astype(np.int32).copy()
        used = np.unique(np.concatenate([self.bt[r, :self.P[r]] for r in range(len(self.P))]))
        self.used = used
        idx = torch.from_numpy(used.astype(np.int64)).to(wl.device)
        self.k = bf16_np(wl.k_pool[:, idx])
        self.v = bf16_np(wl.v_pool[:, idx])
        self.remap = np.full(int(wl.k_pool.shape[1]), -1, dtype=np.int64)
        self.remap[used] = np.arange(used.size)
        self.free_stack = wl.free_stack.cpu().numpy().copy()
        self.free_count = int(wl.free_count.item())
        self.rope = wl.rope.cpu().numpy()
        self.pos = wl.position.cpu().numpy()
        self.slot = wl.slot.cpu().numpy()

    def keys(self, l, h, pages):
        return oracle.gather_row(self.k, l, h, self.remap[np.asarray(pages)])

    def values(self, l, h, pages):
        return oracle.gather_row(self.v, l, h, self.remap[np.asarray(pages)])


def device_rows(pool: torch.Tensor, l: int, h: int, pages) -> np.ndarray:
    """One row chain gathered on the device, copied to the host as uint16."""
    idx = torch.as_tensor(np.asarray(pages, dtype=np.int64), device=pool.device)
    return bf16_np(pool[l, idx, h].reshape(-1, pool.shape[-1]))


def oracle_event(ocfg: OracleConfig, hc: HostCopy, state, qcur, reserve=0, refcount=None,
                 action=None):
    """A1-A9 on host copies; returns a dict of every output.  refcount (host
    int32 per pool page) adds the prefix-preserving steps (target pages
    before the compaction, release after it); action, when given, replaces
    the grant step (actions chosen by the caller)."""
    dem = oracle.demand(ocfg, lambda r, l, h, pages: hc.keys(l, h, pages),
                        hc.bt, hc.P, state, qcur, hc.rope, hc.pos, hc.slot, want_abar=True)
    bt = hc.bt.copy()
    P = hc.P.copy()
    rc = None if refcount is None else np.ascontiguousarray(refcount, np.int32).copy()
    if action is None:
        action, fc, counters = oracle.grow(dem["decision"], bt, P, hc.free_stack,
                                           hc.free_count, reserve, refcount=rc)
    else:
        action = np.ascontiguousarray(action, np.int8)
        fc, counters = hc.free_count, None
    B = len(P)
    # a Shrink action outside the Shrink policy is ignored by the library
    eff = action.copy()
    if ocfg.policy != 1:
        eff[eff == oracle.SHRINK] = oracle.GROW
    ok = np.ones(B, np.uint8)
    copied = 0
    if rc is not None:
        target, ok, copied, fc = oracle.share_plan(eff, bt, P, rc, hc.free_stack, fc)
    dropped = {}
    compacted = {}
    freed = np.zeros(B, np.int32)  # pages of slots each request frees
    for r in range(B):
        m = {oracle.COMPRESS: 1, oracle.SHRINK: 2}.get(int(eff[r]), 0)
        if m == 0 or hc.P[r] < m + 1 or not ok[r]:
            continue
        freed[r] = m
        pages = hc.bt[r, :hc.P[r]]
        for l in range(ocfg.L):
            for h in range(ocfg.Hkv):
                keep = oracle.select(ocfg, dem["abar"][(r, l, h)], pages=m)
                N = keep.size
                dropped[(r, l, h)] = np.nonzero(keep[:N - ocfg.R] == 0)[0].astype(np.int32)
                ks = hc.keys(l, h, pages)
                vs = hc.values(l, h, pages)
                n = oracle.compact(ks, keep)
                oracle.compact(vs, keep)
                compacted[(r, l, h)] = (ks[:n], vs[:n])
    if rc is not None:
        oracle.share_release(bt, target, ok, rc)
    stack = hc.free_stack.copy()
    # only requests that were compressed release a page
    ret = np.where(ok.astype(bool), eff, oracle.COMPRESS).astype(np.int8)
    shrunk, fc = oracle.return_pages(ret, bt, P, stack, fc, refcount=rc)
    return dict(dem=dem, action=action, bt=bt, P=P, free_count=fc, counters=counters,
                dropped=dropped, compacted=compacted, freed=freed, free_stack=stack,
                shrunk=shrunk, ok=ok, copied=copied, refcount=rc)


def row_offsets(P: np.ndarray, L: int, Hkv: int, b: int):
    """Start of each (request, layer, KV head) row in the token-major outputs."""
    offs = {}
    o = 0
    for r in range(len(P)):
        N = int(P[r]) * b
        for l in range(L):
            for h in range(Hkv):
                offs[(r, l, h)] = (o, N)
                o += N
    return offs


def check_decode_after_event(wl, cfg, hc: HostCopy, ref: dict, seed: int, tol: float = 1e-3):
    """One decode step over the cache an event left (block tables, page
    counts and token counts as the GPU event wrote them), every (request,
    layer, KV head) against the fp64 definition of §3.1 Eq. 3 over the
    oracle's rows: its compacted K/V for a request that compressed (freed
    pages of slots), the original rows otherwise.  Returns the worst error
    relative to the row's largest |v|."""
    from paged_kv_cache_04_amd.runner import DecodeRunner
    s = wl.shape
    G = s.Hq // s.Hkv
    pool = gb.Pool(wl.k_pool, wl.v_pool, wl.free_stack, wl.free_count)
    batch = gb.Batch(wl.block_table, wl.num_pages, wl.num_tokens, wl.slot, wl.position,
                     wl.num_pages.cpu().numpy().astype(np.int32).copy())
    dec = DecodeRunner(cfg, pool, batch, wl.rope)
    q = torch.randn((wl.B, s.L, s.Hq, s.d), dtype=torch.float32, device=wl.device,
                    generator=torch.Generator(wl.device).manual_seed(seed))
    outs = [dec.layer(l, q[:, l].contiguous()).cpu().numpy().copy() for l in range(s.L)]
    assert dec.device_errors() == 0
    qn = q.cpu().numpy()
    worst = 0.0
    for r in range(wl.B):
        pages = hc.bt[r, :hc.P[r]]
        for l in range(s.L):
            for h in range(s.Hkv):
                if ref["freed"][r] > 0:
                    keys, vals = ref["compacted"][(r, l, h)]
                else:
                    keys, vals = hc.keys(l, h, pages), hc.values(l, h, pages)
                want, _ = oracle.decode_attention_f64(qn[r, l, h * G:(h + 1) * G], keys, vals,
                                                      hc.rope[int(hc.pos[r])])
                vmax = np.abs(oracle.bf16_to_f64(vals)).max()
                err = np.abs(outs[l][r, h * G:(h + 1) * G].astype(np.float64) - want).max() / vmax
                worst = max(worst, err)
                assert err <= tol, (r, l, h, err)
    return worst
