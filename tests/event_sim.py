"""Successive boundary events on the oracle side, for the multi-event parity
tests.  Test infrastructure: it calls only oracle/ (and the seeded generator
for inputs) and keeps its own state, so nothing the GPU path produced ever
feeds it.

State per tracked (request, layer, KV head) row: the row's K and V in logical
slot order (numpy, bf16 bits), its token count, and per request the summary
state, page count, block table, free stack and position.  One event follows
the library's order: A0 with the current query, A1-A5 over the tracked rows,
A6 (page grant) for the whole batch, A7-A9 for the compressing requests; then
`append` writes the tokens decoded until the next event.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


class OracleEvents:
    def __init__(self, ocfg: oracle.OracleConfig, wl, rows=None):
        """rows: (r, l, h) tracked rows; None tracks every row.  Requests
        with a tracked row keep their summary state.  The decision of a
        request needs all of its rows: it is computed for every request
        whose rows are all tracked (`full_reqs`); with a subset of the
        requests the page grant takes its decisions from
        `decision_override` at event time."""
        self.cfg = ocfg
        s = wl.shape
        self.B = wl.B
        self.all_rows = rows is None
        if rows is None:
            rows = [(r, l, h) for r in range(self.B) for l in range(s.L) for h in range(s.Hkv)]
        self.rows = list(rows)
        self.reqs = sorted({r for r, _, _ in self.rows})
        per_req = {}
        for r, _, _ in self.rows:
            per_req[r] = per_req.get(r, 0) + 1
        self.full_reqs = [r for r in self.reqs if per_req[r] == s.L * s.Hkv]
        self.bt = wl.block_table.cpu().numpy().copy()
        self.P = wl.num_pages.cpu().numpy().astype(np.int32).copy()
        self.N = self.P.astype(np.int64) * s.b
        self.free_stack = wl.free_stack.cpu().numpy().copy()
        self.free_count = int(wl.free_count.item())
        self.pos = wl.position.cpu().numpy().astype(np.int64).copy()
        self.slot = wl.slot.cpu().numpy().copy()
        self.rope = wl.rope.cpu().numpy()
        cap = self.bt.shape[1] * s.b
        self.k = {}
        self.v = {}
        for (r, l, h) in self.rows:
            kk = np.zeros((cap, s.d), dtype=np.uint16)
            vv = np.zeros((cap, s.d), dtype=np.uint16)
            pages = self.bt[r, :self.P[r]]
            ti = torch.from_numpy(np.asarray(pages, dtype=np.int64)).to(wl.device)
            kk[:self.N[r]] = (wl.k_pool[l, ti, h].reshape(-1, s.d).contiguous().cpu()
                              .view(torch.int16).numpy().view(np.uint16))
            vv[:self.N[r]] = (wl.v_pool[l, ti, h].reshape(-1, s.d).contiguous().cpu()
                              .view(torch.int16).numpy().view(np.uint16))
            self.k[(r, l, h)] = kk
            self.v[(r, l, h)] = vv
        self.state = np.zeros((s.L, wl.max_slots, 2, s.Hq, s.d), dtype=np.float32)
        self.t = 0  # next query step to apply

    def ema_until(self, wl, t_end: int):
        """A0 for query steps self.t .. t_end - 1 on the tracked requests."""
        req = np.asarray(self.reqs, dtype=np.int64)
        req_t = torch.from_numpy(req).to(wl.device)
        for t in range(self.t, t_end):
            q = wl.query(t)[req_t].cpu().numpy()
            first = wl.first_step(t)[req_t].cpu().numpy()
            oracle.ema(self.cfg, self.state, np.ascontiguousarray(q), self.slot[req], first)
        self.t = t_end

    def event(self, wl, t_cur: int, reserve: int = 0, decision_override=None):
        """One boundary event whose current query is step t_cur (applied by
        A0 first).  Returns the oracle's outputs for the tracked rows."""
        self.ema_until(wl, t_cur + 1)
        cfg = self.cfg
        G = cfg.G
        qcur = wl.query(t_cur).cpu().numpy()
        qh = {r: oracle.qhat(cfg, self.state, int(self.slot[r]), qcur[r],
                             self.rope[int(self.pos[r])]) for r in self.reqs}

        def score(key):
            r, l, h = key
            q2 = np.ascontiguousarray(qh[r][l][:, h * G:(h + 1) * G])
            return oracle.row(cfg, self.k[key][:self.N[r]], q2)

        with ThreadPoolExecutor(_threads()) as ex:
            res = dict(zip(self.rows, ex.map(score, self.rows)))
        ks = {key: int(v.dp[0]) for key, v in res.items()}
        kl = {key: int(v.dp[1]) for key, v in res.items()}
        out = dict(ks=ks, kl=kl)
        decision = np.zeros(self.B, dtype=np.int8)
        diff = np.zeros(self.B, dtype=np.int64)
        delta = np.zeros(self.B, dtype=np.float64)
        for r in self.full_reqs:
            a = np.array([ks[(r, l, h)] for l in range(cfg.L) for h in range(cfg.Hkv)],
                         dtype=np.int32)
            c = np.array([kl[(r, l, h)] for l in range(cfg.L) for h in range(cfg.Hkv)],
                         dtype=np.int32)
            decision[r], diff[r], delta[r] = oracle.decide(cfg, a, c,
                                                           (int(self.P[r]) - 1) * cfg.b)
        out.update(decision=decision, diff=diff, delta=delta)
        if not self.all_rows:
            decision = np.asarray(decision_override, dtype=np.int8)
        action, self.free_count, counters = oracle.grow(decision, self.bt, self.P,
                                                        self.free_stack, self.free_count, reserve)
        out.update(action=action.copy(), P=self.P.copy(), bt=self.bt.copy(),
                   free_count=self.free_count, counters=counters)

        comp = [key for key in self.rows if action[key[0]] == oracle.COMPRESS]

        def compress(key):
            r = key[0]
            keep = oracle.select(cfg, res[key].abar_all)
            n_old = int(self.N[r])
            dropped = np.nonzero(keep[:n_old - cfg.R] == 0)[0].astype(np.int32)
            n = oracle.compact(self.k[key][:n_old], keep)
            oracle.compact(self.v[key][:n_old], keep)
            return dropped, n

        with ThreadPoolExecutor(_threads()) as ex:
            done = dict(zip(comp, ex.map(compress, comp)))
        out["dropped"] = {key: d for key, (d, _) in done.items()}
        for r in range(self.B):
            if action[r] == oracle.COMPRESS:
                self.N[r] = (int(self.P[r]) - 1) * cfg.b
        return out

    def append(self, k_new: np.ndarray, v_new: np.ndarray):
        """Tokens decoded after the event: k_new/v_new [B][L][Hkv][n][d] bf16
        bits, written at each tracked row's next logical slots."""
        n = k_new.shape[3]
        for (r, l, h) in self.rows:
            o = int(self.N[r])
            self.k[(r, l, h)][o:o + n] = k_new[r, l, h]
            self.v[(r, l, h)][o:o + n] = v_new[r, l, h]
        self.N += n
        self.pos += n

    def row_kv(self, key):
        r = key[0]
        return self.k[key][:self.N[r]], self.v[key][:self.N[r]]
