"""One boundary event over a batch, through the C ABI.

Owns the context, the workspace and the output tensors for a fixed batch
shape, and issues the four library calls in order on one stream:
gp_update_summaries (the current query), gp_demand, gp_grow_page,
gp_compress_hold.  Marshalling only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as gb


class BoundaryRunner:
    def __init__(self, cfg: gb.Config, pool: gb.Pool, batch: gb.Batch, qstate: torch.Tensor,
                 rope: torch.Tensor, want_abar: bool = False, want_dropped: bool = False):
        self.cfg = cfg
        self.ctx = gb.Context(cfg)
        self.pool = pool
        self.batch = batch
        self.qstate = qstate
        self.rope = rope
        dev = qstate.device
        B = batch.block_table.shape[0]
        total_tokens = int(batch.num_pages_host.astype(np.int64).sum()) * cfg.page_size
        max_tokens = int(batch.num_pages_host.max()) * cfg.page_size
        self.total_tokens = total_tokens
        row_tokens = cfg.num_layers * cfg.num_kv_heads * total_tokens
        self.ws = torch.empty(gb.gp_workspace_bytes(self.ctx, B, total_tokens, max_tokens), dtype=torch.uint8,
                              device=dev)
        self.out = gb.DemandOut.empty(cfg, B, dev, row_tokens if want_abar else None)
        self.action = torch.empty(B, dtype=torch.int8, device=dev)
        self.dropped = (torch.full((B, cfg.num_layers, cfg.num_kv_heads,
                                    cfg.page_size * cfg.max_freed), -1,
                                   dtype=torch.int32, device=dev) if want_dropped else None)

    def update(self, q: torch.Tensor, first_step: torch.Tensor, stream=None):
        gb.gp_update_summaries(self.ctx, self.qstate, q, self.batch.slot, first_step, stream)

    def demand(self, q_cur: torch.Tensor, stream=None):
        gb.gp_demand(self.ctx, self.pool, self.batch, self.qstate, q_cur, self.rope, self.ws,
                     self.out, stream)

    def grow(self, decision: torch.Tensor | None = None, reserve_pages: int = 0, stream=None):
        gb.gp_grow_page(self.ctx, self.pool, self.batch,
                        self.out.decision if decision is None else decision, self.action,
                        reserve_pages, stream)

    def compress(self, action: torch.Tensor | None = None, stream=None, all_requests=False):
        act = None if all_requests else (self.action if action is None else action)
        gb.gp_compress_hold(self.ctx, self.pool, self.batch, act, self.ws, self.dropped, stream)

    def event(self, q_cur: torch.Tensor, first_step: torch.Tensor | None = None,
              reserve_pages: int = 0, stream=None):
        """The whole hot path for one batch at its boundary."""
        if first_step is not None:
            self.update(q_cur, first_step, stream)
        self.demand(q_cur, stream)
        self.grow(None, reserve_pages, stream)
        self.compress(None, stream)

    def device_errors(self) -> int:
        return gb.gp_get_device_errors(self.ctx)

    def counters(self) -> dict:
        return gb.gp_get_counters(self.ctx)


class DecodeRunner:
    """Decode-step attention over a batch, one layer per call, through the C
    ABI; owns the workspace and the output for a fixed batch shape."""

    def __init__(self, cfg: gb.Config, pool: gb.Pool, batch: gb.Batch, rope: torch.Tensor,
                 ctx: gb.Context | None = None):
        self.cfg = cfg
        self.ctx = gb.Context(cfg) if ctx is None else ctx
        self.pool = pool
        self.batch = batch
        self.rope = rope
        dev = rope.device
        B = batch.block_table.shape[0]
        self.ws = torch.empty(gb.gp_decode_workspace_bytes(
            self.ctx, B, int(batch.num_pages_host.astype(np.int64).sum())),
            dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32,
                               device=dev)

    def layer(self, layer: int, q: torch.Tensor, qstate: torch.Tensor | None = None,
              first_step: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        gb.gp_decode_attention(self.ctx, self.pool, self.batch, layer, q, qstate, first_step,
                               self.rope, self.out, self.ws, stream)
        return self.out

    def device_errors(self) -> int:
        return gb.gp_get_device_errors(self.ctx)


def sub_batch(batch: gb.Batch, rows) -> gb.Batch:
    """A batch of the given request rows (device copies of their metadata;
    the block tables still name the same pool pages)."""
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=batch.block_table.device)
    return gb.Batch(batch.block_table.index_select(0, idx).contiguous(),
                    batch.num_pages.index_select(0, idx).contiguous(),
                    batch.num_tokens.index_select(0, idx).contiguous(),
                    batch.slot.index_select(0, idx).contiguous(),
                    batch.position.index_select(0, idx).contiguous(),
                    batch.num_pages.index_select(0, idx).cpu().numpy().astype(np.int32).copy())
