"""Seeded synthetic inputs for the boundary event.

This module serves both the GPU path's tests/bench and the oracle's, and holds
none of the method's arithmetic: it draws Gaussians, shuffles pages, builds the
model-side rotary cos/sin cache and stores keys post-rotary (as a model's KV
cache holds them), and applies the model's own per-head query RMSNorm for the
Qwen3-shaped stand-in.  Summary states are never computed here: callers run
the EMA update over the query streams produced here, each side with its own
code.

Workload recipe (stand-ins for the pages' Llama-8B-distill / Qwen3-8B serving
on math and code benchmarks; no dataset item or model weight is used):
  * keys and values: bf16 N(0, 1);
  * per (request, layer, KV head) two orthogonal unit directions u_S, u_L in
    pre-rotary space; the query stream of a KV head's query heads is
    a * u + sigma * noise with a = 0.8 sqrt(d), sigma = 0.6 (RMS about 1), on
    u_L for the older steps and on u_S for the recent ones;
  * planted clusters: c keys per row at random historical slots, equal to
    s * sqrt(d) * rot(pos, u) + 0.1 * noise, where u is the direction the row's
    cluster follows and pos the decoding position of the event: the view whose
    summary follows u concentrates on the cluster, the other stays diffuse;
  * page ids: a seeded permutation of the pool; requests' pages interleave.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 0x6A0F00D


@dataclass(frozen=True)
class ModelShape:
    name: str
    L: int
    Hq: int
    Hkv: int
    d: int = 128
    b: int = 256
    theta: float = 5e5
    qnorm: bool = False


TINY = ModelShape("tiny", L=1, Hq=8, Hkv=2, theta=1e4)
LLAMA8B = ModelShape("llama8b", L=32, Hq=32, Hkv=8, theta=5e5)
QWEN3_8B = ModelShape("qwen3_8b", L=36, Hq=32, Hkv=8, theta=1e6, qnorm=True)


def rope_table(max_pos: int, d: int, theta: float) -> np.ndarray:
    """Model rotary cache [max_pos][d] fp32: cos of the d/2 frequencies, then
    sin; frequency j is theta^(-2j/d) (rotate-half convention), fp64 math."""
    half = d // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0 / d))
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def rotate_keys(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Store a pre-rotary key vector the way the model's cache holds it
    (rotate-half pairing (j, j + d/2)); cos/sin are [d/2]."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def rms_norm_heads(q: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """The Qwen3 per-head query RMSNorm with unit weight (a model step)."""
    return q * torch.rsqrt(q.pow(2).mean(-1, keepdim=True) + eps)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _orthonormal_pair(shape, d, g, device):
    a = torch.randn(*shape, d, generator=g, device=device, dtype=torch.float64)
    b = torch.randn(*shape, d, generator=g, device=device, dtype=torch.float64)
    a = a / a.norm(dim=-1, keepdim=True)
    b = b - (b * a).sum(-1, keepdim=True) * a
    b = b / b.norm(dim=-1, keepdim=True)
    return a.float(), b.float()


@dataclass
class Workload:
    """Device tensors of one boundary scenario (layouts as the C ABI takes them)."""
    shape: ModelShape
    device: torch.device
    k_pool: torch.Tensor          # bf16 [L][pool][Hkv][b][d]
    v_pool: torch.Tensor
    block_table: torch.Tensor     # int32 [B][max_pages]
    num_pages: torch.Tensor       # int32 [B]
    num_tokens: torch.Tensor      # int32 [B]
    slot: torch.Tensor            # int32 [B]
    position: torch.Tensor        # int32 [B]
    free_stack: torch.Tensor      # int32 [pool]
    free_count: torch.Tensor      # int32 [1]
    rope: torch.Tensor            # fp32 [max_pos][d]
    u_short: torch.Tensor         # fp32 [B][L][Hkv][d] query directions
    u_long: torch.Tensor
    max_slots: int
    seed: int
    steps: int                    # EMA steps in the query stream
    short_steps: int              # trailing steps that follow u_short
    meta: dict = field(default_factory=dict)
    # optional schedule of the query stream: (first step, kind) pairs in
    # increasing order, kind in {"long", "short", "diffuse"}; when set it
    # replaces the long-then-short default
    phases: tuple = ()

    @property
    def B(self) -> int:
        return int(self.num_pages.shape[0])

    def query(self, t: int) -> torch.Tensor:
        """Query of EMA step t for every request: fp32 [B][L][Hq][d]
        (normalised, pre-rotary).  Step steps-1 is the current query."""
        s = self.shape
        G = s.Hq // s.Hkv
        g = _gen(self.device, self.seed * 7919 + 1000003 * (t + 1))
        if self.phases:
            kind = [k for t0, k in self.phases if t0 <= t][-1]
        else:
            kind = "short" if t >= self.steps - self.short_steps else "long"
        u = self.u_short if kind == "short" else self.u_long
        base = u.repeat_interleave(G, dim=2)  # [B][L][Hq][d]
        noise = torch.randn(base.shape, generator=g, device=self.device, dtype=torch.float32)
        if kind == "diffuse":
            q = noise  # no preferred direction, RMS 1
        else:
            q = 0.8 * math.sqrt(s.d) * base + 0.6 * noise
        if s.qnorm:
            q = rms_norm_heads(q)
        return q.contiguous()

    def first_step(self, t: int) -> torch.Tensor:
        return torch.full((self.B,), 1 if t == 0 else 0, dtype=torch.uint8, device=self.device)

    def new_tokens(self, event: int, n: int):
        """Keys and values of the n tokens decoded after boundary event
        `event` (0-based), for every request: bf16 N(0, 1), [B][L][Hkv][n][d]
        each.  Seeded per event, independent of what the event did."""
        s = self.shape
        g = _gen(self.device, self.seed * 104729 + 7919 * (event + 1) + 17)
        shp = (self.B, s.L, s.Hkv, n, s.d)
        k = torch.randn(shp, generator=g, device=self.device, dtype=torch.float32)
        v = torch.randn(shp, generator=g, device=self.device, dtype=torch.float32)
        return k.to(torch.bfloat16), v.to(torch.bfloat16)

    def write_tokens(self, r: int, slot0: int, k: torch.Tensor, v: torch.Tensor):
        """Store [L][Hkv][n][d] keys/values of request r at logical slots
        slot0 .. slot0 + n - 1 (within one page) through its block table."""
        b = self.shape.b
        n = k.shape[2]
        assert slot0 % b + n <= b, "appended tokens must stay in one page"
        page = int(self.block_table[r, slot0 // b].item())
        o = slot0 % b
        self.k_pool[:, page, :, o:o + n] = k
        self.v_pool[:, page, :, o:o + n] = v


def make_workload(shape: ModelShape, pages_per_request, pool_pages: int, *, seed: int,
                  device, align=None, cluster_sizes=None, cluster_scale: float = 2.0,
                  free_pages: int = 0, max_pages: int | None = None, steps: int = 1024,
                  short_steps: int = 32, max_slots: int = 512, max_pos: int | None = None,
                  value_pool: bool = True, phases: tuple = ()) -> Workload:
    """Build one scenario.

    pages_per_request: list of P_r (N_r = P_r * b at the boundary).
    align[r] in {"S", "L", None}: which summary direction request r's clusters
    follow (None: no cluster).  cluster_sizes[r]: int or array [L][Hkv].
    free_pages: page ids left on the free stack (taken from unused pool pages).
    """
    device = torch.device(device)
    s = shape
    B = len(pages_per_request)
    P = np.asarray(pages_per_request, dtype=np.int64)
    assert P.sum() + free_pages <= pool_pages, "pool too small"
    if max_pages is None:
        max_pages = int(P.max()) + 8
    rng = np.random.default_rng(seed)
    perm = rng.permutation(pool_pages).astype(np.int32)
    bt = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    # interleave requests' pages: assign the permuted ids round-robin
    owners = np.concatenate([np.full(p, r) for r, p in enumerate(P)])
    rng.shuffle(owners)
    fill = np.zeros(B, dtype=np.int64)
    for idx, r in enumerate(owners):
        bt[r, fill[r]] = perm[idx]
        fill[r] += 1
    off = int(P.sum())
    free = perm[off:off + free_pages].copy()
    free_stack = np.zeros(pool_pages, dtype=np.int32)
    free_stack[:free_pages] = free
    N = P * s.b
    position = N.copy()
    if max_pos is None:
        max_pos = int(position.max()) + 4096
    rope = torch.from_numpy(rope_table(max_pos, s.d, s.theta)).to(device)

    g = _gen(device, seed)
    kshape = (s.L, pool_pages, s.Hkv, s.b, s.d)
    k_pool = torch.empty(kshape, dtype=torch.bfloat16, device=device)
    v_pool = torch.empty(kshape, dtype=torch.bfloat16, device=device)
    used = torch.from_numpy(np.sort(bt[bt >= 0]).astype(np.int64)).to(device)
    for l in range(s.L):
        for pool, _ in ((k_pool, "k"), (v_pool, "v")):
            if pool is v_pool and not value_pool:
                continue
            vals = torch.randn((used.numel(), s.Hkv, s.b, s.d), generator=g, device=device,
                               dtype=torch.float32)
            pool[l].index_copy_(0, used, vals.to(torch.bfloat16))
            del vals
    u_s, u_l = _orthonormal_pair((B, s.L, s.Hkv), s.d, g, device)

    if align is None:
        align = [None] * B
    if cluster_sizes is None:
        cluster_sizes = [8] * B
    bt_t = torch.from_numpy(bt).to(device)
    half = s.d // 2
    for r in range(B):
        if align[r] is None:
            continue
        u = (u_s if align[r] == "S" else u_l)[r]  # [L][Hkv][d]
        cos = rope[int(position[r]), :half]
        sin = rope[int(position[r]), half:]
        ndem = int(N[r]) - s.b
        cs = np.minimum(np.broadcast_to(np.asarray(cluster_sizes[r]), (s.L, s.Hkv)), ndem)
        cs = cs.astype(np.int64)
        slots = np.concatenate([rng.choice(ndem, size=int(cs[l, h]), replace=False)
                                for l in range(s.L) for h in range(s.Hkv)]).astype(np.int64)
        li = np.repeat(np.arange(s.L), cs.sum(axis=1))
        hi = np.concatenate([np.repeat(np.arange(s.Hkv), cs[l]) for l in range(s.L)])
        S = torch.from_numpy(slots).to(device)
        Lt = torch.from_numpy(li.astype(np.int64)).to(device)
        Ht = torch.from_numpy(hi.astype(np.int64)).to(device)
        vec = cluster_scale * math.sqrt(s.d) * u[Lt, Ht] + 0.1 * torch.randn(
            (S.numel(), s.d), generator=g, device=device, dtype=torch.float32)
        vec = rotate_keys(vec, cos, sin).to(torch.bfloat16)
        pages = bt_t[r, S // s.b].long()
        k_pool[Lt, pages, Ht, S % s.b] = vec
        del vec
    i32 = dict(dtype=torch.int32, device=device)
    return Workload(
        shape=s, device=device, k_pool=k_pool, v_pool=v_pool, block_table=bt_t,
        num_pages=torch.tensor(P, **i32), num_tokens=torch.tensor(N, **i32),
        slot=torch.tensor(rng.permutation(max_slots)[:B].astype(np.int32), **i32),
        position=torch.tensor(position, **i32),
        free_stack=torch.from_numpy(free_stack).to(device),
        free_count=torch.tensor([free_pages], **i32), rope=rope,
        u_short=u_s, u_long=u_l, max_slots=max_slots, seed=seed, steps=steps,
        short_steps=short_steps, meta=dict(align=list(align)), phases=tuple(phases))


def tiny(variant: str, device="cpu") -> Workload:
    """1 request, 1 layer, 8 Q / 2 KV heads, d 128, b 256, 4 pages shuffled in
    a 16-page pool; 8 planted keys per KV head at scale 4; 1024 EMA steps.
    variant: "L_grow" (clusters on u_L, free pages), "L_full" (clusters on
    u_L, pool full), "S" (clusters on u_S)."""
    align = {"L_grow": "L", "L_full": "L", "S": "S"}[variant]
    free = 0 if variant == "L_full" else 4
    return make_workload(TINY, [4], 16, seed=SEED_BASE + 0, device=device, align=[align],
                         cluster_sizes=[8], cluster_scale=4.0, free_pages=free, max_pages=8,
                         steps=1024, short_steps=32, max_slots=8)


def _log_uniform_sizes(rng, shape, lo=50, hi=4000):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.int64)


def llama8k(variant: str, device="cuda", pool_pages: int = 4096) -> Workload:
    """Llama-8B shape (32 layers, 32 Q / 8 KV heads, d 128), one request of
    8192 tokens = 32 pages scattered in a pool of pool_pages; per-row clusters
    of log-uniform size in [50, 4000] on the long view ("grow") or the short
    view ("compress")."""
    seed = SEED_BASE + 1
    rng = np.random.default_rng(seed + (0 if variant == "grow" else 17))
    sizes = _log_uniform_sizes(rng, (LLAMA8B.L, LLAMA8B.Hkv))
    return make_workload(LLAMA8B, [32], pool_pages, seed=seed, device=device,
                         align=["L" if variant == "grow" else "S"], cluster_sizes=[sizes],
                         free_pages=8, steps=256, short_steps=32)


def batch64(device="cuda", pool_pages: int = 6144, seed: int = SEED_BASE + 3,
            batch: int = 64, value_pool: bool = True) -> Workload:
    """Continuous-serving snapshot: `batch` requests of Llama-8B shape with page
    counts uniform in [4, 128] (1k-32k tokens), pages interleaved in one pool,
    per request a cluster direction on the long (grow) or short (compress)
    view with log-uniform per-row cluster sizes, and free pages for about a
    third of the growing requests so that the rest fall back."""
    rng = np.random.default_rng(seed)
    P = rng.integers(4, 129, size=batch)
    align = [str(a) for a in rng.choice(["S", "L"], size=batch)]
    free = max(1, sum(a == "L" for a in align) // 3)
    sizes = [_log_uniform_sizes(rng, (LLAMA8B.L, LLAMA8B.Hkv)) for _ in range(batch)]
    return make_workload(LLAMA8B, P.tolist(), pool_pages, seed=seed, device=device, align=align,
                         cluster_sizes=sizes, free_pages=free, max_pages=136, steps=256,
                         short_steps=32, value_pool=value_pool)


EVENT_GAP = 256  # decoded tokens (and summary updates) between two boundary events


def qwen16k_phase(device="cuda", events: int = 10, shape: ModelShape = QWEN3_8B,
                  warmup: int = 1024) -> Workload:
    """Qwen3-8B shape (36 layers, 32 Q / 8 KV heads, query RMSNorm), one
    request of 16384 tokens = 64 pages in a 96-page pool with 16 free pages,
    `events` boundary events EVENT_GAP decoding steps apart.  Per-row clusters
    (log-uniform sizes in [50, 4000]) follow u_L.  Query stream: diffuse for
    `warmup` steps, concentrated on u_L over the first half of the events,
    diffuse again over the second half, so that the short summary first leads
    the long one onto the clusters (Delta < 0) and then leaves them
    (Delta > 0).  Event e (0-based) takes the query of step
    warmup + EVENT_GAP * (e + 1) - 1 as its current query."""
    seed = SEED_BASE + 2
    rng = np.random.default_rng(seed)
    sizes = _log_uniform_sizes(rng, (shape.L, shape.Hkv))
    half = events // 2
    phases = ((0, "diffuse"), (warmup, "long"), (warmup + EVENT_GAP * half, "diffuse"))
    steps = warmup + EVENT_GAP * events
    return make_workload(shape, [64], 96, seed=seed, device=device, align=["L"],
                         cluster_sizes=[sizes], free_pages=16, max_pages=80, steps=steps,
                         max_slots=4, max_pos=16384 + EVENT_GAP * (events + 1) + 16,
                         phases=phases)


def qwen32k_stress(device="cuda", batch: int = 16, shape: ModelShape = QWEN3_8B,
                   warmup: int = 512, events: int = 8) -> Workload:
    """Qwen3-8B shape, `batch` requests of 32768 tokens = 128 pages each, the
    pool exactly their pages (no free page: every Grow falls back), per-row
    log-uniform clusters on u_S or u_L by request, `events` successive
    boundary events EVENT_GAP steps apart after a `warmup`-step stream."""
    seed = SEED_BASE + 4
    rng = np.random.default_rng(seed)
    align = [str(a) for a in rng.choice(["S", "L"], size=batch)]
    sizes = [_log_uniform_sizes(rng, (shape.L, shape.Hkv)) for _ in range(batch)]
    return make_workload(shape, [128] * batch, 128 * batch, seed=seed, device=device,
                         align=align, cluster_sizes=sizes, free_pages=0, max_pages=128,
                         steps=warmup + EVENT_GAP * events, max_slots=batch,
                         max_pos=32768 + EVENT_GAP * (events + 1) + 16)
