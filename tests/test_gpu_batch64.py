"""Parity at full size on the 64-request continuous-serving batch, in the
launch configuration the benchmark times: Llama-8B shape (32 layers, 32
query / 8 KV heads, d 128), page counts uniform in [4, 128], pages
interleaved in a 5120-page pool, free pages for about a third of the growing
requests, one boundary event for all 64 requests.

The oracle cannot score all 16384 (request, layer, KV head) rows within a
test, so it checks a seeded sample of rows one by one, bit for bit: both
D_p values (§3.2 Eq. 2 and Eq. 7), the dropped slots of Eq. 10 and the
compacted K/V bytes.  Its summaries come from running A0 on the sampled
layers only (the update is independent per layer).  Everything else is
checked by properties that hold at any size: the decision is Eq. 8's sign
rule over the request's own D_p values (tau = 0), pages go to the Grow
requests in request order from the top of the free stack while the pool
lasts and the rest fall back (§3.2, App. E.2), every compressing request
ends one page of slots shorter and every growing request keeps its bytes.
The decode step over the same batch (all 32 layers, as the benchmark runs
it) is checked the same way: sampled (request, layer, KV head) outputs
against the fp64 definition of §3.1 Eq. 3, and the summaries it updates on
the sampled layers bit for bit against A0.  Citations are to "GrowPage:
On-Demand KV Budgeting for Efficient LLM Reasoning Serving"."""
import dataclasses
import gc

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_04_amd import synth
from paged_kv_cache_04_amd.runner import DecodeRunner
from gpu_util import device_rows, gb_config, log, oracle_config, run_stream_gpu, runner_for

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU in this container")

POOL_PAGES = 5120      # the benchmark's pool
SAMPLE_LAYERS = 4
ROWS_PER_REQUEST = 2


@needs_gpu
def test_batch64_full_size_sampled_rows():
    log("test_batch64_full_size_sampled_rows")
    gc.collect()
    torch.cuda.empty_cache()
    wl = synth.batch64("cuda", pool_pages=POOL_PAGES)
    s = wl.shape
    G = s.Hq // s.Hkv
    cfg = gb_config(s, max_slots=wl.max_slots)
    ocfg = oracle_config(cfg)
    B = wl.B
    bt0 = wl.block_table.cpu().numpy().copy()
    P0 = wl.num_pages.cpu().numpy().astype(np.int64)
    fs0 = wl.free_stack.cpu().numpy().copy()
    fc0 = int(wl.free_count.item())
    slot = wl.slot.cpu().numpy()
    pos = wl.position.cpu().numpy()
    rope = wl.rope.cpu().numpy()
    b, R = ocfg.b, ocfg.R

    rng = np.random.default_rng(6464)
    layers = np.sort(rng.choice(s.L, SAMPLE_LAYERS, replace=False))
    sample = [(r, int(rng.choice(layers)), int(rng.integers(s.Hkv)))
              for r in range(B) for _ in range(ROWS_PER_REQUEST)]
    pre = {}
    for r, l, h in sample:
        pages = bt0[r, :P0[r]]
        pre[(r, l, h)] = (device_rows(wl.k_pool, l, h, pages), device_rows(wl.v_pool, l, h, pages))
    log(f"  {len(sample)} sampled rows over layers {layers.tolist()}, "
        f"{int(P0.sum())} pages in use, {fc0} free")

    run = runner_for(wl, cfg, want_abar=False, want_dropped=True)
    q_cur = run_stream_gpu(run, wl)
    run.demand(q_cur)
    run.grow()
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() == 0

    # the oracle's summaries of the sampled layers (A0 acts per layer)
    ocfg_s = dataclasses.replace(ocfg, L=SAMPLE_LAYERS)
    state = np.zeros((SAMPLE_LAYERS, wl.max_slots, 2, s.Hq, s.d), np.float32)
    lidx = torch.as_tensor(layers, device="cuda")
    qs = None
    for t in range(wl.steps):
        qs = wl.query(t).index_select(1, lidx).cpu().numpy()
        oracle.ema(ocfg_s, state, qs, slot, wl.first_step(t).cpu().numpy())

    o = run.out
    ks = o.k_short.cpu().numpy()
    kl = o.k_long.cpu().numpy()
    diff = o.k_diff.cpu().numpy()
    decision = o.decision.cpu().numpy()
    action = run.action.cpu().numpy()
    bt = run.batch.block_table.cpu().numpy()
    P = run.batch.num_pages.cpu().numpy()
    nt = run.batch.num_tokens.cpu().numpy()
    dropped = run.dropped.cpu().numpy()

    # Eq. 8 at tau = 0 over each request's own D_p values
    want_diff = (ks.astype(np.int64) - kl.astype(np.int64)).sum(axis=(1, 2))
    assert np.array_equal(diff, want_diff)
    assert np.array_equal(decision, np.where(want_diff > 0, oracle.GROW, oracle.COMPRESS))
    # grant in request order from the top of the free stack, then fallback
    fc = fc0
    want_action = np.zeros(B, np.int8)
    want_bt, want_P = bt0.copy(), P0.copy()
    for r in range(B):
        if decision[r] == oracle.GROW and fc > 0:
            fc -= 1
            want_bt[r, want_P[r]] = fs0[fc]
            want_P[r] += 1
            want_action[r] = 1
    assert np.array_equal(action, want_action)
    assert np.array_equal(P, want_P) and np.array_equal(bt, want_bt)
    assert int(wl.free_count.item()) == fc
    grown = action == 1
    fallback = (decision == oracle.GROW) & ~grown
    log(f"  {int(grown.sum())} grown, {int(fallback.sum())} fell back, "
        f"{int((decision == oracle.COMPRESS).sum())} chose Compress & Hold")
    assert grown.any() and fallback.any() and (decision == oracle.COMPRESS).any()
    assert np.array_equal(nt, np.where(grown, P0 * b, (P0 - 1) * b))

    # sampled rows against the oracle, bit for bit
    qh_cache = {}
    n_comp = 0
    for r, l, h in sample:
        if r not in qh_cache:
            qh_cache[r] = oracle.qhat(ocfg_s, state, int(slot[r]), qs[r], rope[int(pos[r])])
        li = int(np.searchsorted(layers, l))
        q2 = np.ascontiguousarray(qh_cache[r][li][:, h * G:(h + 1) * G])
        k_pre, v_pre = pre[(r, l, h)]
        res = oracle.row(ocfg, k_pre, q2)
        assert (ks[r, l, h], kl[r, l, h]) == (res.dp[0], res.dp[1]), (r, l, h)
        N = int(P0[r]) * b
        if grown[r]:
            assert np.all(dropped[r, l, h] == -1)
            assert np.array_equal(device_rows(wl.k_pool, l, h, bt0[r, :P0[r]]), k_pre), (r, l, h)
            assert np.array_equal(device_rows(wl.v_pool, l, h, bt0[r, :P0[r]]), v_pre), (r, l, h)
            continue
        n_comp += 1
        keep = oracle.select(ocfg, res.abar_all)
        want_drop = np.nonzero(keep[:N - R] == 0)[0]
        assert np.array_equal(dropped[r, l, h, :b], want_drop), (r, l, h)
        kw, vw = k_pre.copy(), v_pre.copy()
        n = oracle.compact(kw, keep)
        oracle.compact(vw, keep)
        assert n == N - b
        kg = device_rows(wl.k_pool, l, h, bt[r, :P[r]])[:n]
        vg = device_rows(wl.v_pool, l, h, bt[r, :P[r]])[:n]
        assert np.array_equal(kg, kw[:n]) and np.array_equal(vg, vw[:n]), (r, l, h)
    log(f"  {len(sample)} rows match ({n_comp} compacted)")
    del run, wl, pre
    gc.collect()
    torch.cuda.empty_cache()


DEC_TOL = 1e-3  # of the row's largest |v|: fp32 arithmetic, hardware exp2


@needs_gpu
def test_batch64_decode_sampled_heads():
    log("test_batch64_decode_sampled_heads")
    gc.collect()
    torch.cuda.empty_cache()
    wl = synth.batch64("cuda", pool_pages=POOL_PAGES)
    s = wl.shape
    G = s.Hq // s.Hkv
    cfg = gb_config(s, max_slots=wl.max_slots)
    ocfg = oracle_config(cfg)
    B = wl.B
    bt = wl.block_table.cpu().numpy()
    P = wl.num_pages.cpu().numpy().astype(np.int64)
    slot = wl.slot.cpu().numpy()
    pos = wl.position.cpu().numpy()
    rope = wl.rope.cpu().numpy()
    rng = np.random.default_rng(6465)
    layers = np.sort(rng.choice(s.L, SAMPLE_LAYERS, replace=False))
    sample = [(r, int(rng.choice(layers)), int(rng.integers(s.Hkv)))
              for r in range(B) for _ in range(ROWS_PER_REQUEST)]

    # summaries up to the decode step, then one decode step of every layer
    run = runner_for(wl, cfg, want_abar=False, want_dropped=False)
    run_stream_gpu(run, wl, steps=wl.steps - 1)
    q = wl.query(wl.steps - 1)
    no_first = torch.zeros(B, dtype=torch.uint8, device="cuda")
    dec = DecodeRunner(cfg, run.pool, run.batch, wl.rope)
    outs = {}
    for l in range(s.L):
        o = dec.layer(l, q[:, l].contiguous(), run.qstate, no_first)
        if l in layers:
            outs[l] = o.cpu().numpy().copy()
    torch.cuda.synchronize()
    assert dec.device_errors() == 0

    # A0 on the sampled layers: the stream, then the decode step's update
    ocfg_s = dataclasses.replace(ocfg, L=SAMPLE_LAYERS)
    state = np.zeros((SAMPLE_LAYERS, wl.max_slots, 2, s.Hq, s.d), np.float32)
    lidx = torch.as_tensor(layers, device="cuda")
    for t in range(wl.steps):
        first = wl.first_step(t).cpu().numpy() if t < wl.steps - 1 else no_first.cpu().numpy()
        oracle.ema(ocfg_s, state, wl.query(t).index_select(1, lidx).cpu().numpy(), slot, first)
    got_state = run.qstate.index_select(0, lidx).cpu().numpy()
    assert np.array_equal(got_state.view(np.uint32), state.view(np.uint32))

    qn = q.index_select(1, lidx).cpu().numpy()
    worst = 0.0
    for r, l, h in sample:
        pages = bt[r, :P[r]]
        keys = device_rows(wl.k_pool, l, h, pages)
        vals = device_rows(wl.v_pool, l, h, pages)
        li = int(np.searchsorted(layers, l))
        want, _ = oracle.decode_attention_f64(qn[r, li, h * G:(h + 1) * G], keys, vals,
                                              rope[int(pos[r])])
        vmax = np.abs(oracle.bf16_to_f64(vals)).max()
        err = np.abs(outs[l][r, h * G:(h + 1) * G].astype(np.float64) - want).max() / vmax
        worst = max(worst, err)
        assert err <= DEC_TOL, (r, l, h, err)
    log(f"  {len(sample)} sampled heads, worst error / max|v| = {worst:.2e}; summaries of "
        f"layers {layers.tolist()} bit-exact")
    del run, dec, wl
    gc.collect()
    torch.cuda.empty_cache()
