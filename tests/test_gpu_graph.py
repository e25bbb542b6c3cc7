"""The boundary event captured in a HIP graph: the library's calls enqueue
only kernels on the caller's stream (no allocation, memset or host
synchronisation), so a caller can record gp_update_summaries, gp_demand,
gp_grow_page and gp_compress_hold once and replay them.  Each replay starts
from the same restored state (eager copies, synchronised, between replays)
and must reproduce the eager event bit for bit: D_p, decisions, grants,
block tables, token counts, distributions, dropped slots and every pool
byte."""
import numpy as np
import pytest
import torch

from paged_kv_cache_04_amd import synth
from gpu_util import gb_config, log, run_stream_gpu, runner_for

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU in this container")

SMALL = synth.ModelShape("small", L=2, Hq=8, Hkv=2, theta=1e4)


def bits(t: torch.Tensor) -> torch.Tensor:
    """Integer view for bitwise comparison (unused pool pages may hold NaN
    patterns, which a value comparison calls unequal)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.float64:
        return t.view(torch.int64)
    return t


@needs_gpu
def test_event_replayed_from_a_graph_matches_eager():
    log("test_event_replayed_from_a_graph_matches_eager")
    P = [3, 6, 2, 5, 4, 7]
    align = ["L", "S", "L", "L", "S", "L"]
    wl = synth.make_workload(SMALL, P, 40, seed=7400, device="cuda", align=align,
                             cluster_sizes=[30] * len(P), free_pages=2, steps=80,
                             short_steps=16, max_slots=8)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q_prev = run_stream_gpu(run, wl, steps=wl.steps - 1)
    assert q_prev is not None
    q_cur = wl.query(wl.steps - 1)
    first = torch.zeros(wl.B, dtype=torch.uint8, device="cuda")
    state = [wl.k_pool, wl.v_pool, wl.block_table, wl.num_pages, wl.num_tokens, wl.free_stack,
             wl.free_count, run.qstate, run.dropped]
    saved = [x.clone() for x in state]

    def restore():
        for dst, src in zip(state, saved):
            dst.copy_(src)
        torch.cuda.synchronize()

    def event():
        run.update(q_cur, first)
        run.demand(q_cur)
        run.grow()
        run.compress()

    o = run.out
    outputs = lambda: [o.k_short, o.k_long, o.k_diff, o.delta, o.decision, o.abar, run.action,
                       wl.block_table, wl.num_pages, wl.num_tokens, wl.free_stack,
                       wl.free_count, run.qstate, run.dropped, wl.k_pool, wl.v_pool]

    event()
    torch.cuda.synchronize()
    assert run.device_errors() == 0
    eager = [x.clone() for x in outputs()]
    action = run.action.cpu().numpy()
    log(f"  eager actions {action.tolist()}")
    assert (action == 1).any() and (action == 0).any()

    restore()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        event()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        # eager work of the program's own between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert run.device_errors() == 0
        for i, (a, b) in enumerate(zip(eager, outputs())):
            assert torch.equal(bits(a), bits(b)), (rep, i)
    log("  3 replays identical to the eager event")
    del g
