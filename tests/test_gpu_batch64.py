"""Parity at full size on the 64-request continuous-serving batch, in the
launch configuration the benchmark times: Llama-8B shape (32 layers, 32
query / 8 KV heads, d 128), page counts uniform in [4, 128], pages
interleaved in a 5120-page pool, free pages for about a third of the growing
requests, one boundary event for all 64 requests.

Every one of the 16384 (request, layer, KV head) rows is checked against the
oracle, bit for bit: the summaries after the query stream (A0), both D_p
values of every row (§3.2 Eq. 2 and Eq. 7), each request's Delta, integer
difference and decision from the oracle's own D_p (Eq. 8), the page grants
and fallbacks in request order (§3.3, §4.2), the dropped slots of every
compressing row (§3.3 Eq. 10) and every K/V byte each row holds afterwards:
the kept rows in slot order for a compressing request, the untouched rows
for a growing one.  The oracle runs one layer at a time on host copies
(tests/batch_oracle.py), keeping digests of the expected bytes.
The decode step over the same batch (all 32 layers, as the benchmark runs
it) is checked on sampled (request, layer, KV head) outputs against the fp64
definition of §3.1 Eq. 3, and the summaries it updates on the sampled layers
bit for bit against A0.  Citations are to "GrowPage: On-Demand KV Budgeting
for Efficient LLM Reasoning Serving"."""
import dataclasses
import gc

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_04_amd import synth
from paged_kv_cache_04_amd.runner import DecodeRunner
from batch_oracle import StreamedBatchOracle
from gpu_util import (device_rows, gb_config, log, oracle_config, run_stream_gpu,
                      run_stream_oracle, runner_for)

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU in this container")

POOL_PAGES = 5120      # the benchmark's pool
SAMPLE_LAYERS = 4
ROWS_PER_REQUEST = 2


@needs_gpu
@pytest.mark.timeout(900)
def test_batch64_full_size_every_row():
    log("test_batch64_full_size_every_row")
    gc.collect()
    torch.cuda.empty_cache()
    wl = synth.batch64("cuda", pool_pages=POOL_PAGES)
    s = wl.shape
    cfg = gb_config(s, max_slots=wl.max_slots)
    ocfg = oracle_config(cfg)
    B, b, R = wl.B, ocfg.b, ocfg.R
    bt0 = wl.block_table.cpu().numpy().copy()
    P0 = wl.num_pages.cpu().numpy().astype(np.int64)
    fs0 = wl.free_stack.cpu().numpy().copy()
    fc0 = int(wl.free_count.item())
    slot = wl.slot.cpu().numpy()
    log(f"  {int(P0.sum())} pages in use, {fc0} free, {B * s.L * s.Hkv} rows")

    run = runner_for(wl, cfg, want_abar=False, want_dropped=True)
    q_cur = run_stream_gpu(run, wl)
    torch.cuda.synchronize()
    # A0 over the whole stream, every layer, against the oracle
    state, q_last = run_stream_oracle(wl, ocfg)
    got_state = run.qstate.cpu().numpy()
    assert np.array_equal(got_state[:, slot].view(np.uint32), state[:, slot].view(np.uint32))
    del got_state
    log("  summaries bit-exact")

    ref = StreamedBatchOracle(ocfg, wl, state, q_last, bt0, P0, log=log)
    ref.before()

    run.demand(q_cur)
    run.grow()
    run.compress()
    torch.cuda.synchronize()
    assert run.device_errors() == 0

    o = run.out
    np.testing.assert_array_equal(o.k_short.cpu().numpy(), ref.ks)
    np.testing.assert_array_equal(o.k_long.cpu().numpy(), ref.kl)
    want = ref.decide_and_grow(fs0, fc0)
    np.testing.assert_array_equal(o.k_diff.cpu().numpy(), want["diff"])
    np.testing.assert_array_equal(o.delta.cpu().numpy(), want["delta"])
    np.testing.assert_array_equal(o.decision.cpu().numpy(), want["decision"])
    action = run.action.cpu().numpy()
    np.testing.assert_array_equal(action, want["action"])
    np.testing.assert_array_equal(run.batch.block_table.cpu().numpy(), want["bt"])
    np.testing.assert_array_equal(run.batch.num_pages.cpu().numpy(), want["P"])
    assert int(wl.free_count.item()) == want["free_count"]
    c = run.counters()
    assert (c["grown"], c["compress"], c["fallback"]) == tuple(int(x) for x in want["counters"])
    grown = action == oracle.GROW
    fallback = (want["decision"] == oracle.GROW) & ~grown
    log(f"  D_p of every row, decisions and grants match: {int(grown.sum())} grown, "
        f"{int(fallback.sum())} fell back, "
        f"{int((want['decision'] == oracle.COMPRESS).sum())} chose Compress & Hold")
    assert grown.any() and fallback.any() and (want["decision"] == oracle.COMPRESS).any()
    np.testing.assert_array_equal(run.batch.num_tokens.cpu().numpy(),
                                  np.where(grown, P0 * b, (P0 - 1) * b))

    dropped = run.dropped.cpu().numpy()
    for r in range(B):
        for l in range(s.L):
            for h in range(s.Hkv):
                if grown[r]:
                    assert np.all(dropped[r, l, h] == -1), (r, l, h)
                else:
                    np.testing.assert_array_equal(dropped[r, l, h, :b], ref.dropped[(r, l, h)],
                                                  err_msg=str((r, l, h)))
    log("  dropped slots of every compressing row match")
    n_comp, n_grow = ref.after(action)
    log(f"  K/V bytes of {n_comp} compacted and {n_grow} untouched rows match")
    ref.copier.release()
    del run, wl, ref
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
