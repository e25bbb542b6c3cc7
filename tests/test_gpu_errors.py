"""Error paths on the GPU, each forced from the host with inputs that the
kernels' own checks catch (every kernel still runs to completion and no
access leaves its buffers): the device error bits are set and the pool is left
as it was where the event cannot proceed.  Calls that host-side validation
refuses return an error status and enqueue nothing.  The in-place
compaction's only ordering hazard is checked by running it with several
persistent grid sizes (a different workgroup-to-item order each)."""
import numpy as np
import pytest
import torch

from paged_kv_cache_04_amd import binding as gb
from paged_kv_cache_04_amd import synth
from gpu_util import device_rows, gb_config, log, run_stream_gpu, runner_for

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU in this container")

SMALL = synth.ModelShape("small", L=2, Hq=8, Hkv=2, theta=1e4)
ERR_SLOT, ERR_POSITION, ERR_PAGE, ERR_SHORT, ERR_PAGES, ERR_LONG = 1, 2, 4, 8, 16, 64
ONE_HEAD = synth.ModelShape("one-head", L=1, Hq=4, Hkv=1, theta=1e4)


def _workload(seed):
    return synth.make_workload(SMALL, [4, 3], 16, seed=seed, device="cuda", align=["L", "S"],
                               cluster_sizes=[20, 20], free_pages=0, steps=40, short_steps=8,
                               max_slots=4)


@needs_gpu
def test_page_id_out_of_range():
    """A block-table entry beyond the pool: scoring reads a valid page in its
    place and flags PAGE; compaction of that request leaves its pages alone."""
    log("test_page_id_out_of_range")
    wl = _workload(41)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    good = wl.block_table[0, :4].cpu().numpy().copy()
    k_before = device_rows(wl.k_pool, 1, 1, good)
    wl.block_table[0, 2] = wl.k_pool.shape[1] + 5
    run.demand(q)
    run.grow()
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() & ERR_PAGE
    assert int(run.action[0].item()) == 0  # pool full: fallback to compression
    assert np.array_equal(device_rows(wl.k_pool, 1, 1, good), k_before)


@needs_gpu
def test_slot_and_position_out_of_range():
    """A summary slot beyond the pool and a position beyond the rotary table:
    the EMA update skips the request, calibration uses a zero scale and a
    clamped position, and both bits are raised."""
    log("test_slot_and_position_out_of_range")
    wl = _workload(42)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    state_before = run.qstate.clone()
    wl.slot[1] = wl.max_slots
    wl.position[0] = wl.rope.shape[0] + 3
    run.update(q, wl.first_step(wl.steps))
    run.demand(q)
    torch.cuda.synchronize()
    bits = run.device_errors()
    assert bits & ERR_SLOT and bits & ERR_POSITION, bits
    # request 0's slot was updated, nothing else changed
    s0 = int(wl.slot[0].item())
    diff = (run.qstate != state_before).any(dim=(0, 2, 3, 4)).cpu().numpy()
    assert diff[s0] and diff.sum() == 1


@needs_gpu
def test_stale_host_page_counts():
    """The host mirror of the page counts disagrees with the device: the plan
    rejects the batch, PAGES is raised, and no later kernel of the event runs
    (outputs and pool untouched)."""
    log("test_stale_host_page_counts")
    wl = _workload(43)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    run.batch.num_pages_host[0] += 1
    run.out.k_short.fill_(-7)
    pages = wl.block_table[1, :3].cpu().numpy().copy()
    k_before = device_rows(wl.k_pool, 0, 0, pages)
    run.ws = torch.empty(gb.gp_workspace_bytes(run.ctx, 2, 8 * 256, 5 * 256), dtype=torch.uint8,
                         device="cuda")
    run.demand(q)
    run.grow(decision=torch.zeros(2, dtype=torch.int8, device="cuda"))
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() & ERR_PAGES
    assert (run.out.k_short == -7).all()
    assert np.array_equal(device_rows(wl.k_pool, 0, 0, pages), k_before)


@needs_gpu
@pytest.mark.parametrize("dev_pages", [(0, 7), (5, 2)])
def test_device_page_counts_outside_limits(dev_pages):
    """Device page counts whose total agrees with the host mirror but which
    break a limit: a count of 0, or a count longer than the workspace's
    per-row rings (sized from the host mirror's longest request, 4 pages).
    The plan rejects the batch, PAGES is raised, and no later kernel of the
    event touches the outputs or the pool."""
    log(f"test_device_page_counts_outside_limits {dev_pages}")
    wl = _workload(44)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    assert list(run.batch.num_pages_host) == [4, 3]
    wl.num_pages.copy_(torch.tensor(dev_pages, dtype=torch.int32, device="cuda"))
    run.out.k_short.fill_(-7)
    pages = wl.block_table[1, :3].cpu().numpy().copy()
    k_before = device_rows(wl.k_pool, 0, 0, pages)
    run.demand(q)
    run.grow(decision=torch.zeros(2, dtype=torch.int8, device="cuda"))
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() & ERR_PAGES
    assert (run.out.k_short == -7).all()
    assert np.array_equal(device_rows(wl.k_pool, 0, 0, pages), k_before)


@needs_gpu
def test_host_validation_errors():
    """Calls that host-side validation refuses return an error status and
    enqueue nothing: a workspace smaller than gp_workspace_bytes, Compress &
    Hold without the preceding gp_demand on that workspace (or with another
    workspace), a decode workspace smaller than gp_decode_workspace_bytes,
    a layer outside the model; the pool, token counts and outputs keep
    their contents."""
    log("test_host_validation_errors")
    wl = _workload(44)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    torch.cuda.synchronize()
    pages = wl.block_table[1, :3].cpu().numpy().copy()
    k_before = device_rows(wl.k_pool, 0, 0, pages)
    nt_before = wl.num_tokens.clone()
    run.out.k_short.fill_(-7)
    small = torch.empty(run.ws.numel() - 256, dtype=torch.uint8, device="cuda")

    def refused(fn, what):
        with pytest.raises(gb.GPError, match=what):
            fn()

    refused(lambda: gb.gp_demand(run.ctx, run.pool, run.batch, run.qstate, q, run.rope, small,
                                 run.out), "workspace")
    # no gp_demand has prepared this context's workspace yet
    refused(lambda: gb.gp_compress_hold(run.ctx, run.pool, run.batch, None, run.ws), "workspace")
    run.demand(q)
    other = torch.empty_like(run.ws)
    refused(lambda: gb.gp_compress_hold(run.ctx, run.pool, run.batch, None, other), "workspace")
    torch.cuda.synchronize()
    assert (run.out.k_short != -7).all()  # the accepted gp_demand ran
    assert np.array_equal(device_rows(wl.k_pool, 0, 0, pages), k_before)
    assert torch.equal(wl.num_tokens, nt_before)
    # decode: workspace and layer checks
    total_pages = int(run.batch.num_pages_host.sum())
    need = gb.gp_decode_workspace_bytes(run.ctx, wl.B, total_pages)
    out = torch.zeros((wl.B, wl.shape.Hq, wl.shape.d), dtype=torch.float32, device="cuda")
    q0 = q[:, 0].contiguous()
    refused(lambda: gb.gp_decode_attention(
        run.ctx, run.pool, run.batch, 0, q0, None, None, run.rope, out,
        torch.empty(need - 256, dtype=torch.uint8, device="cuda")), "workspace")
    refused(lambda: gb.gp_decode_attention(
        run.ctx, run.pool, run.batch, wl.shape.L, q0, None, None, run.rope, out,
        torch.empty(need, dtype=torch.uint8, device="cuda")), "invalid argument")
    torch.cuda.synchronize()
    assert (out == 0).all()
    assert run.device_errors() == 0


@needs_gpu
@pytest.mark.parametrize("groups", [1, 3, 64])
def test_compaction_grid_sizes_give_identical_bytes(groups):
    """The compaction's persistent grid takes its (row, K/V) items in a
    different workgroup order for every grid size; in-place compaction must
    not depend on it: the pool, token counts and dropped slots are bitwise
    those of the default grid."""
    log(f"test_compaction_grid_sizes_give_identical_bytes[{groups}]")
    P = [7, 3, 9, 5, 4]
    results = []
    for g in (0, groups):
        wl = synth.make_workload(SMALL, P, 40, seed=4500, device="cuda",
                                 align=["S", "S", "L", "S", "S"], cluster_sizes=[40] * 5,
                                 free_pages=0, steps=80, short_steps=16, max_slots=8)
        cfg = gb_config(wl.shape, max_slots=wl.max_slots, compact_workgroups=g)
        run = runner_for(wl, cfg)
        q = run_stream_gpu(run, wl)
        run.event(q)
        torch.cuda.synchronize()
        assert run.device_errors() == 0
        bt = wl.block_table.cpu().numpy()
        used = torch.as_tensor(np.unique(bt[bt >= 0]), device="cuda")
        results.append((wl.k_pool[:, used].view(torch.int16).clone(),
                        wl.v_pool[:, used].view(torch.int16).clone(),
                        wl.num_tokens.clone(), run.dropped.clone()))
        del run, wl
    for a, b in zip(results[0], results[1]):
        assert torch.equal(a, b)


@needs_gpu
def test_compress_skips_request_beyond_selection_limit():
    """A request longer than the 65536 tokens the selection takes, whose
    decision is Compress & Hold in an event where the grant step has already
    given another request a page, is left as it was (LONG bit, same bytes
    and token count), while the rest of the batch is compressed or grown as
    the oracle says: nothing is refused half-way through an event."""
    from gpu_util import HostCopy, oracle_config, oracle_event, run_stream_oracle
    log("test_compress_skips_request_beyond_selection_limit")
    P = [257, 5, 3]
    wl = synth.make_workload(ONE_HEAD, P, 268, seed=4250, device="cuda", align=["S", "S", "L"],
                             cluster_sizes=[30, 30, 30], free_pages=1, steps=60, short_steps=8,
                             max_slots=4)
    cfg = gb_config(wl.shape, max_slots=wl.max_slots)
    hc = HostCopy(wl)
    run = runner_for(wl, cfg)
    q = run_stream_gpu(run, wl)
    k0 = device_rows(wl.k_pool, 0, 0, hc.bt[0, :P[0]])
    v0 = device_rows(wl.v_pool, 0, 0, hc.bt[0, :P[0]])
    run.demand(q)
    run.grow()
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() == ERR_LONG
    ocfg = oracle_config(cfg)
    state, qcur = run_stream_oracle(wl, ocfg)
    ref = oracle_event(ocfg, hc, state, qcur)
    action = run.action.cpu().numpy()
    log(f"  actions {action.tolist()}")
    np.testing.assert_array_equal(action, ref["action"])
    assert action[0] == 0  # the long request was to compress
    np.testing.assert_array_equal(run.out.k_short.cpu().numpy(), ref["dem"]["ks"])
    np.testing.assert_array_equal(run.out.k_long.cpu().numpy(), ref["dem"]["kl"])
    np.testing.assert_array_equal(wl.block_table.cpu().numpy(), ref["bt"])
    np.testing.assert_array_equal(wl.num_pages.cpu().numpy(), ref["P"])
    nt = wl.num_tokens.cpu().numpy()
    assert nt[0] == P[0] * 256
    assert np.array_equal(device_rows(wl.k_pool, 0, 0, hc.bt[0, :P[0]]), k0)
    assert np.array_equal(device_rows(wl.v_pool, 0, 0, hc.bt[0, :P[0]]), v0)
    dropped = run.dropped.cpu().numpy()
    assert np.all(dropped[0] == -1)
    for r in (1, 2):
        if action[r] != 0:
            assert nt[r] == P[r] * 256 and np.all(dropped[r] == -1)
            continue
        np.testing.assert_array_equal(dropped[r, 0, 0, :256], ref["dropped"][(r, 0, 0)])
        k_want, v_want = ref["compacted"][(r, 0, 0)]
        n = k_want.shape[0]
        assert nt[r] == n
        pages = hc.bt[r, :hc.P[r]]
        assert np.array_equal(device_rows(wl.k_pool, 0, 0, pages)[:n], k_want)
        assert np.array_equal(device_rows(wl.v_pool, 0, 0, pages)[:n], v_want)
