"""The oracle over every row of a large batch, streamed one layer at a time.

Test infrastructure: it calls only oracle/ (and torch for device-to-host
copies of the inputs).  A batch whose K and V do not fit in host memory is
checked in two passes over the layers:

  before the event, for each layer: copy that layer's K and V of the pages
  the batch uses to pinned host buffers, and for every (request, KV head)
  row compute both D_p (§3.2 Eq. 2 and Eq. 7), the slots Eq. 10 drops
  (§3.3), and digests of the bytes the row must hold afterwards: its kept
  rows in slot order (if it compresses) and its original rows (if it grows);

  after the event, for each layer: copy the same pages again and digest
  what the GPU left in each row.

Only the per-row D_p values, dropped slots and 16-byte digests are kept,
so host memory stays at two layers' worth of pinned K and V.  Citations are
to "GrowPage: On-Demand KV Budgeting for Efficient LLM Reasoning Serving".
"""
from __future__ import annotations

import hashlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle


def digest(a: np.ndarray) -> bytes:
    return hashlib.blake2b(np.ascontiguousarray(a).tobytes(), digest_size=16).digest()


class LayerCopier:
    """Copies one layer's K and V of a fixed page set into pinned host
    buffers: [U][Hkv][b][d] uint16 views, U = number of pages."""

    def __init__(self, wl, pages: np.ndarray):
        s = wl.shape
        self.wl = wl
        self.idx = torch.as_tensor(np.asarray(pages, np.int64), device=wl.device)
        shp = (len(pages), s.Hkv, s.b, s.d)
        self.k = torch.empty(shp, dtype=torch.bfloat16, pin_memory=True)
        self.v = torch.empty(shp, dtype=torch.bfloat16, pin_memory=True)
        self.k_np = self.k.view(torch.int16).numpy().view(np.uint16)
        self.v_np = self.v.view(torch.int16).numpy().view(np.uint16)

    def load(self, layer: int):
        for src, dst in ((self.wl.k_pool, self.k), (self.wl.v_pool, self.v)):
            tmp = src[layer].index_select(0, self.idx)
            dst.copy_(tmp)
            del tmp
        torch.cuda.synchronize()

    def release(self):
        del self.k, self.v, self.k_np, self.v_np


class StreamedBatchOracle:
    """Expected outputs of one boundary event for every row of a batch.

    ocfg: the oracle's method parameters; state: the oracle's summary pool
    after the query stream; qcur: host [B][L][Hq][d] current queries;
    bt, P: host block tables and page counts at the event."""

    def __init__(self, ocfg: oracle.OracleConfig, wl, state, qcur, bt, P, threads: int = 16,
                 log=print):
        self.cfg = ocfg
        self.wl = wl
        self.bt = np.asarray(bt)
        self.P = np.asarray(P).astype(np.int64)
        self.B = len(self.P)
        self.threads = threads
        self.log = log
        rope = wl.rope.cpu().numpy()
        pos = wl.position.cpu().numpy()
        slot = wl.slot.cpu().numpy()
        self.qh = [oracle.qhat(ocfg, state, int(slot[r]), qcur[r], rope[int(pos[r])])
                   for r in range(self.B)]
        self.pages = np.unique(np.concatenate([self.bt[r, :self.P[r]] for r in range(self.B)]))
        self.remap = {int(p): i for i, p in enumerate(self.pages)}
        L, H = ocfg.L, ocfg.Hkv
        self.ks = np.zeros((self.B, L, H), np.int32)
        self.kl = np.zeros((self.B, L, H), np.int32)
        self.dropped = {}
        self.want_compacted = {}
        self.want_original = {}
        self.copier = LayerCopier(wl, self.pages)

    def _row_pages(self, r: int) -> np.ndarray:
        return np.array([self.remap[int(p)] for p in self.bt[r, :self.P[r]]], np.int64)

    def _rows(self, arr: np.ndarray, r: int, h: int) -> np.ndarray:
        t = arr[self._row_pages(r), h]  # [P][b][d]
        return np.ascontiguousarray(t.reshape(-1, t.shape[-1]))

    def before(self):
        """Score, select and digest every row, layer by layer (call before
        the event changes K and V)."""
        cfg = self.cfg
        G = cfg.G
        for l in range(cfg.L):
            self.copier.load(l)

            def work(rh, l=l):
                r, h = rh
                keys = self._rows(self.copier.k_np, r, h)
                vals = self._rows(self.copier.v_np, r, h)
                q2 = np.ascontiguousarray(self.qh[r][l][:, h * G:(h + 1) * G])
                res = oracle.row(cfg, keys, q2)
                keep = oracle.select(cfg, res.abar_all).astype(bool)
                N = keys.shape[0]
                drop = np.nonzero(~keep[:N - cfg.R])[0].astype(np.int32)
                comp = (digest(keys[keep]), digest(vals[keep]))
                orig = (digest(keys), digest(vals))
                return (r, l, h), res.dp, drop, comp, orig

            jobs = [(r, h) for r in range(self.B) for h in range(cfg.Hkv)]
            with ThreadPoolExecutor(self.threads) as ex:
                for key, dp, drop, comp, orig in ex.map(work, jobs):
                    self.ks[key], self.kl[key] = int(dp[0]), int(dp[1])
                    self.dropped[key] = drop
                    self.want_compacted[key] = comp
                    self.want_original[key] = orig
            if l % 8 == 7:
                self.log(f"    oracle: layers 0..{l} scored and selected")

    def decide_and_grow(self, free_stack, free_count: int, reserve: int = 0):
        """A5 per request from the oracle's own D_p, then A6 over the batch."""
        cfg = self.cfg
        B = self.B
        decision = np.zeros(B, np.int8)
        diff = np.zeros(B, np.int64)
        delta = np.zeros(B, np.float64)
        for r in range(B):
            decision[r], diff[r], delta[r] = oracle.decide(cfg, self.ks[r], self.kl[r],
                                                           (int(self.P[r]) - 1) * cfg.b,
                                                           int(self.P[r]))
        bt = self.bt.astype(np.int32).copy()
        P = self.P.astype(np.int32).copy()
        action, fc, counters = oracle.grow(decision, bt, P, np.asarray(free_stack, np.int32),
                                           int(free_count), reserve)
        return dict(decision=decision, diff=diff, delta=delta, action=action, bt=bt, P=P,
                    free_count=fc, counters=counters)

    def after(self, action: np.ndarray):
        """Digest what each row holds after the event and compare: a
        compressing row's first (P - 1) b slots are its kept rows in slot
        order; a growing row still holds its original rows.  Returns the
        number of rows compared of each kind."""
        cfg = self.cfg
        n_comp = n_grow = 0
        for l in range(cfg.L):
            self.copier.load(l)

            def work(rh, l=l):
                r, h = rh
                keys = self._rows(self.copier.k_np, r, h)
                vals = self._rows(self.copier.v_np, r, h)
                key = (r, l, h)
                if action[r] == oracle.COMPRESS:
                    n = keys.shape[0] - cfg.b
                    got = (digest(keys[:n]), digest(vals[:n]))
                    return key, got == self.want_compacted[key], True
                got = (digest(keys), digest(vals))
                return key, got == self.want_original[key], False

            jobs = [(r, h) for r in range(self.B) for h in range(cfg.Hkv)]
            with ThreadPoolExecutor(self.threads) as ex:
                for key, ok, comp in ex.map(work, jobs):
                    assert ok, f"K/V bytes of row {key} differ from the oracle's"
                    n_comp += comp
                    n_grow += not comp
            if l % 8 == 7:
                self.log(f"    K/V of layers 0..{l} match")
        return n_comp, n_grow
