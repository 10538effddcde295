"""Benchmark of the BeaconKV eviction hot path on one MI355X.

One step = one eviction period of the whole path over the full batch:
  1. the cache grows back to L by the period's 128 decode steps: fresh
     synthetic K/V rows are copied into rows [B, L) (from a pre-generated
     pool, never repeating a row still cached) and the length is reset,
  2. bkv_fps_update ingests the period's 128 pre-RoPE queries per query head
     (Continual FPS, shrinking buffers that fill),
  3. bkv_score selects beacons, rotates observation rows and scores every
     cached key,
  4. bkv_select keeps the window plus the top B_KV - W,
  5. bkv_compact gathers the kept K/V rows in place.

Workload: all 36 layers of Qwen3-4B (32 query / 8 KV heads, d = 128) at batch
16, bf16, evicting 2176 -> 2048 (window 32, 16 recent + 16 beacons, buffer
128 -> 16), seeded synthetic data.  Inputs are resident in HBM before timing.

Three schedules of the same passes are timed.  Serial: every stage on one
stream, in order (stage times and the roofline come from it: each kernel runs
alone).  Overlapped: the ingest and beacon FPS of pass i + 1 run on a second
stream while pass i scores, selects and compacts, as a decode loop would feed
the buffers while the cache is being evicted.  Pipelined (the reported
throughput): as overlapped, with the slots in three groups whose scorings take
turns, so one group compacts while the other scores.  Events keep every data
dependency.

Prints one JSON line (see the keys below).  --gpus N > 1 is refused: this
build targets one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_eviction_continual_amd import bkv, configs, synth  # noqa: E402

HBM_PEAK_GBPS = 8000.0
NORTH_STAR_FRAC = 0.60  # score + compaction pass: fraction of peak HBM bandwidth aimed for
CFG = 3             # the benchmark workload (qwen3-4b-36layers-b16-B2048); 4 and 5 on request
POOL_MAX = 64       # distinct 128-step query blocks (0.6 GB each at the default workload) cycled over the steps
POOL_BYTES = 60e9   # cap on the query-block pool of the larger workloads
N_EVENTS = 240      # evictions in a 32K-token generation (first at L = 2176)
APPEND_BLOCKS = 4   # pre-generated blocks of new tokens' K/V rows, appended at [B, L) before every pass
APPEND_BYTES = 24e9 # cap on that pool (the largest workload holds two blocks)


def kernel_source_hash() -> str:
    """Hash of the HIP sources with comments and blank lines removed, so that
    recorded counter figures stay tied to the code they were measured on."""
    import re

    h = hashlib.sha256()
    for name in ("fps.hip", "score.hip", "select.hip", "bkv_api.hip", "bkv_device.hpp", "fps_full.hip", "decode.hip"):
        with open(os.path.join(ROOT, "kv_cache_eviction_continual_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def append_plan(t: int, n_blocks: int, N: int, a: int, e: int):
    """Copies that give slots [a, e) their new tokens of pass t: slot s takes
    slot (s + r) % N of pool block t % n_blocks, r = (t // n_blocks) % N, so a
    (block, rotation) pair comes back only after n_blocks * N passes.  Returns
    (first destination slot, first source slot, count) runs of contiguous
    slots."""
    rot = (t // n_blocks) % N
    runs = []
    s = a
    while s < e:
        src = (s + rot) % N
        n = min(e - s, N - src)
        runs.append((s, src, n))
        s += n
    return runs


class State:
    """Device-resident state of the metric workload."""

    def __init__(self, w, dev, n_pool):
        self.w = w
        self.n_pool = n_pool
        N, Hq, Hkv, d = w.n_slots, w.n_q_heads, w.n_kv_heads, w.head_dim
        self.N = N
        syn = synth.Synth(w, seed=0, device=dev)
        self.syn = syn
        log("generating K/V %s x 2 and %d query blocks" % ((N, Hkv, w.max_len, d), n_pool))
        self.K = syn.keys()
        self.V = syn.values()
        # every decode period brings new queries: the pool holds the blocks of
        # global periods [pool_first, pool_first + n_pool), regenerated before
        # every timed phase for that phase's periods, so no phase re-ingests a
        # block an earlier one ingested (a re-ingested query would duplicate a
        # buffered one and turn FPS rounds into exact ties)
        self.pool_first = 0
        self.blocks = [syn.query_block(b) for b in range(n_pool)]
        R = w.n_recent
        self.recent = [blk[:, :, -R:].contiguous() for blk in self.blocks]
        self.shape = bkv.make_shape(N, Hkv, Hq, d, w.max_len, self.K.dtype)
        self.ws = bkv.alloc_workspace(self.shape, R, w.n_beacons, device=dev)
        self.qbuf = torch.zeros(N, Hq, w.capacity, d, dtype=self.K.dtype, device=dev)
        self.qcount = torch.zeros(N, Hq, dtype=torch.int32, device=dev)
        self.len_full = torch.full((N,), w.length, dtype=torch.int32, device=dev)
        self.length = self.len_full.clone()
        # the tokens of every decode period are new: pass t writes fresh K/V rows at [B, L) (block t % P of
        # the pool, the pool's slots rotated by t // P, so that no appended row repeats one still cached); a
        # pass that only reset the length would find stale copies of earlier rows there, whose exact ties
        # with their originals push every eviction to the tail and shrink the compaction pass by pass
        n_new = w.length - w.budget
        blk_bytes = 2 * N * Hkv * n_new * d * self.K.element_size()
        self.n_append = max(2, min(APPEND_BLOCKS, int(APPEND_BYTES // blk_bytes)))
        self.new_k = [syn.keys(max_len=n_new, block=1 + b) for b in range(self.n_append)]
        self.new_v = [syn.values(max_len=n_new, block=1 + b) for b in range(self.n_append)]
        self.pass_base = 0  # pass t = pass_base + i; advanced after every timed phase
        self.scores = torch.empty(N, Hkv, w.max_len, dtype=torch.float32, device=dev)
        self.kept = torch.empty(N, Hkv, w.budget, dtype=torch.int32, device=dev)
        now0 = w.length - 1
        ev = np.arange(N_EVENTS)
        pos_now = (now0 + w.interval * ev).astype(np.int32)
        self.pos_now = torch.from_numpy(np.repeat(pos_now[:, None], N, axis=1)).to(dev).contiguous()
        rp = pos_now[:, None] - np.arange(R - 1, -1, -1)[None, :]
        self.recent_pos = torch.from_numpy(np.repeat(rp[:, None, :], N, axis=1).astype(np.int32)).to(dev).contiguous()
        # warm the buffers with the first L queries of the stream (17 periods)
        self.n_warm = w.warm_steps // w.interval
        for b in range(self.n_warm):
            blk = self.blocks[b] if b < n_pool else syn.query_block(b)
            bkv.bkv_fps_update(self.shape, blk, blk.shape[2], self.qbuf, self.qcount, w.capacity, w.shrink_to, self.ws)
            del blk
        torch.cuda.synchronize()
        self.refresh_blocks(0)

    def period(self, i):
        """Global decode period of pass i of the current phase (the warm-up
        periods come first)."""
        return self.n_warm + self.pass_base + i

    def block(self, i):
        """Pool index of pass i's query block.  Within a phase of at most
        n_pool passes every pass has a block of its own; longer phases wrap
        around the pool (and then re-ingest queries the buffers may hold)."""
        return (self.period(i) - self.pool_first) % self.n_pool

    def event(self, i):
        """Index of pass i in the simulated generation's eviction events
        (positions of the recent queries and of the current step)."""
        return (self.pass_base + i) % N_EVENTS

    def refresh_blocks(self, n_passes):
        """Regenerates the pool for the next phase's periods (outside any
        timed region): blocks of global periods period(0) ... period(0) +
        n_pool - 1 (a phase of n_passes passes also primes period n_passes)."""
        first = self.period(0)
        if first == self.pool_first:
            return
        self.pool_first = first
        R = self.w.n_recent
        for k in range(self.n_pool):
            self.blocks[k] = None
            self.recent[k] = None
        for k in range(self.n_pool):
            self.blocks[k] = self.syn.query_block(first + k)
            self.recent[k] = self.blocks[k][:, :, -R:].contiguous()
        # the blocks are generated on the current stream; the schedules' own
        # streams read them, so the generation must be complete first
        if self.blocks[0].is_cuda:
            torch.cuda.synchronize()
        if n_passes + 1 > self.n_pool:
            log("phase of %d passes over a pool of %d query blocks: blocks wrap around" % (n_passes, self.n_pool))

    def append_new_tokens(self, i, g):
        """The decode period's new tokens: fresh K/V rows at [B, L) of group g's slots (enqueued on the current
        stream)."""
        w = self.w
        t = self.pass_base + i
        nk, nv = self.new_k[t % self.n_append], self.new_v[t % self.n_append]
        B, L = w.budget, w.length
        for dst, src, n in append_plan(t, self.n_append, self.N, g.sl.start, g.sl.stop):
            self.K[dst:dst + n, :, B:L].copy_(nk[src:src + n])
            self.V[dst:dst + n, :, B:L].copy_(nv[src:src + n])

    def ingest(self, i, g, stream):
        w = self.w
        bkv.bkv_fps_update(g.shape, self.blocks[self.block(i)][g.sl], w.interval, self.qbuf[g.sl], self.qcount[g.sl],
                           w.capacity, w.shrink_to, g.ws, stream=stream)

    def picks(self, g, stream):
        w = self.w
        bkv.bkv_beacon_picks(g.shape, self.qbuf[g.sl], self.qcount[g.sl], w.capacity, w.n_recent, w.n_beacons, g.ws,
                             stream=stream)

    def score_picked(self, i, g, stream):
        w = self.w
        p, e = self.block(i), self.event(i)
        bkv.bkv_score_picked(g.shape, self.K[g.sl], self.length[g.sl], self.recent[p][g.sl], self.recent_pos[e][g.sl],
                             w.n_recent, w.n_beacons, self.pos_now[e][g.sl], w.rope_theta, self.scores[g.sl], g.ws,
                             stream=stream)

    def group_workspace(self, key):
        """A workspace of its own for a group of slots (cached per key)."""
        if not hasattr(self, "_ws_cache"):
            self._ws_cache = {}
        if key not in self._ws_cache:
            n = key[1] - key[0]
            shape = bkv.make_shape(n, self.w.n_kv_heads, self.w.n_q_heads, self.w.head_dim, self.w.max_len,
                                   self.K.dtype)
            self._ws_cache[key] = bkv.alloc_workspace(shape, self.w.n_recent, self.w.n_beacons, device=self.K.device)
        return self._ws_cache[key]


class Group:
    """A contiguous range [a, b) of sequence slots with its own workspace and
    streams.  Slots are independent units of the whole path, so a group is
    just the library called on that range (every tensor is slot-major)."""

    def __init__(self, st, a, b, ws, main, side):
        w = st.w
        self.sl = slice(a, b)
        self.shape = bkv.make_shape(b - a, w.n_kv_heads, w.n_q_heads, w.head_dim, w.max_len, st.K.dtype)
        self.ws, self.main, self.side = ws, main, side
        self.ready = None     # beacon FPS of the group's next pass, enqueued on its side stream
        self.scored = None    # the group's last scoring
        self.released = None  # what the group's next beacon FPS waits for (its scoring, or its compaction)


HEAD_STAGES = ("grow", "fps_update", "beacon_picks", "score")


class Schedule:
    """Enqueues eviction passes i = 0, 1, ... in order.

    grow(i, g) appends the decode period's new tokens to group g's slots and
    resets their cache length (the hole-filling phase also writes positions),
    tail(i, rec, g) selects and compacts it; both run on the group's main
    stream.  Serial: one group (every slot) and one stream; ingest and scoring
    (beacon FPS included) of pass i run there too, in order.  Overlapped: a
    side stream per group (default priority) runs the ingest and then the
    beacon FPS of pass i + 1 while the main stream scores, selects and
    compacts pass i.  The ingest only follows pass i's beacon FPS (same
    stream; scoring reads copies of the picked rows, not the buffers); the
    beacon FPS of pass i + 1 waits for pass i's scoring (the reader of the
    picks), or with picks_after_tail for its compaction, and pass i + 1's
    scoring waits for it.  A compaction workgroup fills a CU's registers, so
    an FPS wave on a CU keeps compaction blocks off it: started after the
    compaction, the beacon FPS runs beside the next pass's new-token append
    instead (measured faster for the order-preserving layout, whose
    compaction is long; the hole-filling layout's short one-call tail keeps
    the earlier start).  With several groups
    (pipelined), each group has its own main stream and workspace (the side
    stream is shared), and the groups' scorings take turns (each waits for
    the previous one), so one group's selection and compaction run beside the
    next group's scoring.
    Every pass does the same work in every schedule (bkv_beacon_picks then
    bkv_score_picked, which together are bkv_score).  `ev` is a dict of
    (start, end) event pairs per stage, recorded for group 0, or None."""

    def __init__(self, st, grow, tail, overlap, tail_stages=("select", "compact"), groups=1, picks_after_tail=False):
        self.st, self.grow, self.tail, self.overlap = st, grow, tail, overlap
        self.tail_stages = tail_stages
        self.picks_after_tail = picks_after_tail
        assert overlap or groups == 1
        # serial: the current stream.  Overlapped: every group on a stream of its own and one side stream for
        # all groups, all taken from torch's pool in a row, none of them the current (default) stream: a process
        # has only four hardware queues, and a stream that shares one with another busy stream is serialised
        # behind it (measured: successive schedules that left group 0 on the default stream alternated between
        # about 3.0 and 3.5 ms per pass as the pool handed out streams on other queues)
        cur = torch.cuda.current_stream()
        side = torch.cuda.Stream() if overlap else None
        bounds = [st.N * k // groups for k in range(groups + 1)]
        self.groups = []
        for k in range(groups):
            a, b = bounds[k], bounds[k + 1]
            ws = st.ws if groups == 1 else st.group_workspace((a, b))
            self.groups.append(Group(st, a, b, ws, torch.cuda.Stream() if overlap else cur, side))
        # the new streams start after everything already enqueued on the current one
        for s in {g.main for g in self.groups} | ({side} if side is not None else set()):
            if s != cur:
                s.wait_stream(cur)
        self.last_scored = None

    @property
    def workspaces(self):
        return [g.ws for g in self.groups]

    def _side_work(self, i, g, ev):
        side = g.side
        if ev is not None:
            ev["fps_update"][0].record(side)
        self.st.ingest(i, g, side)
        if ev is not None:
            ev["fps_update"][1].record(side)
        if g.released is not None:
            side.wait_event(g.released)
        if ev is not None:
            ev["beacon_picks"][0].record(side)
        self.st.picks(g, side)
        if ev is not None:
            ev["beacon_picks"][1].record(side)
        g.ready = torch.cuda.Event()
        g.ready.record(side)

    def prime(self, i):
        """Enqueues pass i's ingest and beacon FPS ahead of time (overlapped schedules)."""
        if not self.overlap:
            return
        for g in self.groups:
            if g.ready is None:
                g.scored = torch.cuda.Event()
                g.scored.record(g.main)
                g.released = g.scored
                self._side_work(i, g, None)

    def run(self, i, ev=None):
        st = self.st
        self.prime(i)
        for k, g in enumerate(self.groups):
            m = g.main
            e = ev if k == 0 else None
            rec = (lambda name, j: e[name][j].record(m)) if e is not None else (lambda name, j: None)
            if self.overlap:
                m.wait_event(g.ready)
            if self.last_scored is not None and len(self.groups) > 1:
                m.wait_event(self.last_scored)
            with torch.cuda.stream(m):
                rec("grow", 0)
                self.grow(i, g)
                rec("grow", 1)
                if not self.overlap:
                    rec("fps_update", 0)
                    st.ingest(i, g, m)
                    rec("fps_update", 1)
                    rec("beacon_picks", 0)
                    st.picks(g, m)
                    rec("beacon_picks", 1)
                rec("score", 0)
                st.score_picked(i, g, m)
                rec("score", 1)
                if self.overlap:
                    g.scored = torch.cuda.Event()
                    g.scored.record(m)
                    self.last_scored = g.scored
                    if not self.picks_after_tail:
                        g.released = g.scored
                        self._side_work(i + 1, g, e)  # measured as this pass's ingest and beacon FPS stages
                self.tail(i, rec, g)
                if self.overlap and self.picks_after_tail:
                    # the next beacon FPS waits for the compaction (whose workgroups fill whole CUs) and runs
                    # beside the next pass's new-token append; the ingest still overlaps the scoring
                    g.released = torch.cuda.Event()
                    g.released.record(m)
                    self._side_work(i + 1, g, e)


def new_events(sched):
    names = HEAD_STAGES
    return {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for n in names + sched.tail_stages}


def timed_passes(sched, warmup, steps):
    """warmup untimed passes, then `steps` timed ones between two device
    synchronisations; returns (seconds, per-stage mean ms, per-stage spread,
    rows moved by the timed passes)."""
    sched.st.refresh_blocks(warmup + steps)
    for i in range(warmup):
        sched.run(i)
    sched.prime(warmup)  # the first timed pass's ingest stays outside the timed region
    torch.cuda.synchronize()
    for ws in sched.workspaces:
        bkv.bkv_reset_device_status(ws)
    evs = [new_events(sched) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sched.run(warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for ws in sched.workspaces:
        status = bkv.bkv_read_device_status(ws)
        assert status == 0, "device status %d" % status
    rows_moved = sum(bkv.ws_rows_moved(ws) for ws in sched.workspaces)
    stage_ms = {n: float(np.mean([e[n][0].elapsed_time(e[n][1]) for e in evs])) for n in evs[0]}
    # the next phase appends other new tokens and ingests other query blocks;
    # an overlapped schedule has already ingested the block of the pass after
    # its last one
    sched.st.pass_base += warmup + steps + (1 if sched.overlap else 0)
    return elapsed, stage_ms, spread(evs, sched), rows_moved


def spread(evs, sched):
    """p10 / median / p90 (ms) of every stage over the timed passes, and of
    the main stream's span of a pass (grow start to the last tail stage's end)."""
    def pct(xs):
        return [float(v) for v in np.percentile(xs, [10, 50, 90])]

    out = {n: pct([e[n][0].elapsed_time(e[n][1]) for e in evs]) for n in evs[0]}
    last = sched.tail_stages[-1]
    out["pass_main_stream"] = pct([e["grow"][0].elapsed_time(e[last][1]) for e in evs])
    return out


def time_hole_fill(st, warmup, steps, overlap, groups=1):
    """The same eviction pass in the hole-filling layout (rows carry their
    positions; only kept rows beyond the budget move).  Runs on the state the
    order-preserving phase left; each pass first appends the positions of the
    interval's new tokens at rows [B, L)."""
    w = st.w
    N, Hkv, B, L = st.N, w.n_kv_heads, w.budget, w.length
    dev = st.K.device
    pos = torch.arange(w.max_len, dtype=torch.int32, device=dev).expand(N, Hkv, w.max_len).contiguous()
    new_rows = L - B
    # positions of the new tokens of pass i: above every earlier one
    fresh = [torch.full((N, Hkv, new_rows), w.max_len + new_rows * i, dtype=torch.int32, device=dev)
             + torch.arange(new_rows, dtype=torch.int32, device=dev) for i in range(min(steps + warmup, 64))]

    def grow(i, g):
        st.length[g.sl].copy_(st.len_full[g.sl])
        st.append_new_tokens(i, g)
        pos[g.sl, :, B:L].copy_(fresh[i % len(fresh)][g.sl] + new_rows * len(fresh) * (i // len(fresh)))

    def tail(i, rec, g):
        rec("select_compact", 0)
        bkv.bkv_select_compact_fill(g.shape, st.scores[g.sl], st.K[g.sl], st.V[g.sl], pos[g.sl], st.length[g.sl], B,
                                    w.window, st.kept[g.sl], g.ws)
        rec("select_compact", 1)

    sched = Schedule(st, grow, tail, overlap, ("select_compact",), groups=groups)
    elapsed, stage_ms, stage_spread, rows_moved = timed_passes(sched, warmup, steps)
    row_bytes = w.head_dim * 2
    moved_per_pass = rows_moved / steps                       # K and V rows
    compact_bytes = moved_per_pass * row_bytes * 2 + moved_per_pass / 2 * 4 * 2  # rows + positions, read + write
    units = N * Hkv
    score_bytes = units * (L * row_bytes + w.obs_rows * row_bytes + L * 4)
    sc_ms = stage_ms["score"] + stage_ms["select_compact"]
    return {
        "layout": "hole-filling (rows carry positions; kept rows beyond the budget fill the evicted rows below it)",
        "score_compact": {
            "what": "score + one-call selection and hole filling: algorithmic bytes (K read once, observation rows, "
                    "scores; moved rows and positions read and written) / the two stages' HIP-event time",
            "algorithmic_bytes": score_bytes + compact_bytes,
            "ms": sc_ms,
            "GBps": (score_bytes + compact_bytes) / (sc_ms * 1e6),
            "frac_of_peak": (score_bytes + compact_bytes) / (sc_ms * 1e6) / HBM_PEAK_GBPS,
        },
        "passes_per_s": steps / elapsed,
        "ms_per_step": elapsed * 1e3 / steps,
        "stage_ms": stage_ms,
        "stage_ms_p10_p50_p90": stage_spread,
        "rows_moved_per_pass": moved_per_pass,
        "compact_algorithmic_bytes": compact_bytes,
        "note": "select_compact is bkv_select_compact_fill: selection and hole filling in one kernel",
    }


def copy_probe(dev, nbytes=1 << 30, reps=10):
    """Bandwidth of a plain device copy of known size (read + write bytes)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms, "GBps": 2 * nbytes / ms / 1e6}


class OracleSample:
    """Inputs of randomly sampled (slot, KV head) units of the workload, as
    numpy storage arrays, for timing the CPU oracle.  Each unit's query heads
    get an untimed warm-up ingest of three periods (48 live rows, so the timed
    period ends at 64, the mean live count of the steady state)."""

    def __init__(self, st: State, warm_blocks: int = 3, seed: int = 1234):
        self.st, self.w = st, st.w
        self.warm_blocks = warm_blocks
        self.rng = np.random.default_rng(seed)
        self.units = []
        self._blocks = {}
        self._full = {}

    def _full_block(self, b):
        """Query block b of the stream (the first periods: the pool now holds later ones)."""
        if b not in self._full:
            self._full[b] = self.st.syn.query_block(b)
        return self._full[b]

    def _block(self, b, n, g0):
        key = (b, n, g0)
        if key not in self._blocks:
            self._blocks[key] = synth.to_numpy_storage(self._full_block(b)[n:n + 1, g0:g0 + self.w.group])
        return self._blocks[key]

    def add(self):
        import oracle

        st, w = self.st, self.w
        G = w.group
        n, h = int(self.rng.integers(0, st.N)), int(self.rng.integers(0, w.n_kv_heads))
        g0 = h * G
        qbuf = np.zeros((1, G, w.capacity, w.head_dim), dtype=np.uint16)
        qcount = np.zeros((1, G), dtype=np.int32)
        for b in range(self.warm_blocks):
            oracle.fps_update(self._block(b, n, g0), qbuf, qcount, w.shrink_to)
        p, e = self.warm_blocks, 0
        u = {"K": synth.to_numpy_storage(st.K_pristine[n, h]), "V": synth.to_numpy_storage(st.V_pristine[n, h]),
             "qbuf": qbuf, "qcount": qcount, "blk": self._block(p, n, g0),
             "recent": synth.to_numpy_storage(self._full_block(p)[n, g0:g0 + G, -w.n_recent:]),
             "rpos": st.recent_pos[e, n].cpu().numpy(), "pos_now": int(st.pos_now[e, n])}
        self.units.append(u)
        return u

    def run(self, u, fresh: bool):
        """One unit: ingest of the period's block, beacon FPS and scoring at
        L, selection, compaction of K and V.  fresh=True works on copies (the
        unit can be run again); the copies are inside the returned time."""
        import oracle

        w = self.w
        t0 = time.perf_counter()
        if fresh:
            K, V, qbuf, qcount = u["K"].copy(), u["V"].copy(), u["qbuf"].copy(), u["qcount"].copy()
        else:
            K, V, qbuf, qcount = u["K"], u["V"], u["qbuf"], u["qcount"]
        oracle.fps_update(u["blk"], qbuf, qcount, w.shrink_to)
        s, _, _, _ = oracle.score_unit(K, w.length, u["recent"], u["rpos"], qbuf[0], qcount[0], w.n_beacons,
                                       u["pos_now"], w.rope_theta)
        kept = oracle.select(s, w.length, w.budget, w.window)
        oracle.compact(K, kept)
        oracle.compact(V, kept)
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_build() -> str:
    import oracle

    return "gcc " + " ".join(oracle.BUILD_FLAGS)


def cpu_baseline(sample: OracleSample, budget_s: float = 10.0, min_units: int = 4, max_units: int = 1024):
    """The CPU oracle (single-threaded C, binary64) on a bounded sample of
    units: each is run once, on its own inputs (prepared untimed), with the
    calling thread pinned to one host core for the duration."""
    st, w = sample.st, sample.w
    allowed = sorted(os.sched_getaffinity(0))
    core = allowed[0]
    os.sched_setaffinity(0, {core})  # pid 0: the calling thread, which runs the oracle's C calls
    try:
        done, t_total = 0, 0.0
        while done < max_units:
            u = sample.add()
            fresh = dict(u, K=u["K"].copy(), V=u["V"].copy(), qbuf=u["qbuf"].copy(), qcount=u["qcount"].copy())
            t_total += sample.run(fresh, fresh=False)
            done += 1
            if done >= min_units and t_total >= budget_s:
                break
    finally:
        os.sched_setaffinity(0, allowed)
    per_unit = t_total / done
    units_per_pass = st.N * w.n_kv_heads
    return {
        "value": 1.0 / (per_unit * units_per_pass),
        "unit": "passes/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "%d (slot, KV head) units of the workload, each: ingest of one 128-query block for its %d query "
                  "heads, beacon FPS, scoring at L=%d, selection and compaction; %.1f s of oracle time "
                  "(%.3f s per unit), extrapolated to %d units per pass" % (done, w.group, w.length, t_total,
                                                                           per_unit, units_per_pass),
        "pinned_core": core,
        "host_threads_available": len(allowed),
        "cpu_model": cpu_model(),
        "oracle_build": oracle_build(),
    }


def host_threads(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_baseline_all_cores(sample: OracleSample, budget_s: float = 10.0, threads: int = 0):
    """The same oracle on every host thread at once: the units are
    independent, so T threads each run sampled units (on fresh copies of
    their inputs; the oracle's C calls release the interpreter lock) until
    the time budget is spent.  Rate = units finished / wall time."""
    import threading

    st, w = sample.st, sample.w
    T = threads or host_threads()
    units = sample.units
    assert units, "run cpu_baseline first: it prepares the sampled units"
    counter = [0]
    lock = threading.Lock()
    t_start = time.perf_counter()
    deadline = t_start + budget_s

    def worker():
        while time.perf_counter() < deadline:
            with lock:
                k = counter[0]
                counter[0] += 1
            sample.run(units[k % len(units)], fresh=True)

    pool = [threading.Thread(target=worker) for _ in range(T)]
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    wall = time.perf_counter() - t_start
    done = counter[0]
    units_per_pass = st.N * w.n_kv_heads
    return {
        "value": done / wall / units_per_pass,
        "unit": "passes/s",
        "cores": T,
        "kind": "oracle",
        "sample": "%d unit runs over %d threads in %.1f s of wall time, cycling over the %d sampled units of the "
                  "single-core baseline (fresh copies of their inputs, copies included), extrapolated to %d units "
                  "per pass" % (done, T, wall, len(units), units_per_pass),
        "cpu_model": cpu_model(),
        "oracle_build": oracle_build(),
    }


def covering_radius_deg(hist, beacons, heads_per_batch=8):
    """Per head: the largest angle (degrees) from any row of the history to
    its nearest beacon (the k-centre objective FPS greedily minimises).
    hist [N, Hq, n, d] and beacons [N, Hq, k, d] storage tensors; returns a
    float64 array [N, Hq].  A reported statistic, evaluated in fp32 with torch."""
    N, Hq, n, d = hist.shape
    out = np.empty((N, Hq))
    for s in range(N):
        for g0 in range(0, Hq, heads_per_batch):
            X = hist[s, g0:g0 + heads_per_batch].float()
            X = X / X.norm(dim=-1, keepdim=True).clamp_min(1e-12)
            B = beacons[s, g0:g0 + heads_per_batch].float()
            B = B / B.norm(dim=-1, keepdim=True).clamp_min(1e-12)
            cos = torch.bmm(X, B.transpose(1, 2).contiguous()).amax(dim=-1)      # nearest beacon per row
            worst = cos.amin(dim=-1).clamp(-1.0, 1.0)                            # farthest row per head
            out[s, g0:g0 + heads_per_batch] = torch.rad2deg(torch.arccos(worst)).double().cpu().numpy()
    return out


def fps_compare(reps: int = 3):
    """Naive full-history FPS against Continual FPS on one layer of the
    Qwen3-14B workload (batch 32, 40 query heads: 1,280 heads) over a
    32,768-query generation with an eviction every 128 steps: time per
    eviction and over the generation, memory, and the beacons' covering
    radius at the end.  Prints its own JSON line."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bkv.load()
    w = configs.get(5)
    N, Hq, d, n = w.batch, w.n_q_heads, w.head_dim, 32768
    k, C, M, T = w.n_beacons, w.capacity, w.shrink_to, w.interval
    heads = N * Hq
    events = n // T
    log("generating the %d-query history of %d heads" % (n, heads))
    syn = synth.Synth(w, n_slots=N, seed=0, device=dev)
    blocks = [syn.query_block(b) for b in range(events)]
    hist = torch.cat(blocks, dim=2).contiguous()
    es = hist.element_size()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, r):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(r):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / r

    # naive: FPS over the whole history so far, at several history lengths
    naive = {}
    picks = torch.empty(N, Hq, k, dtype=torch.int32, device=dev)
    ws_full = torch.empty(bkv.bkv_fps_full_workspace_size(bkv.make_shape(N, 1, Hq, d, n, hist.dtype), n),
                          dtype=torch.uint8, device=dev)
    for m in (4096, 8192, 16384, n):
        h = hist if m == n else hist[:, :, :m].contiguous()
        shape = bkv.make_shape(N, 1, Hq, d, m, hist.dtype)
        ms = timed(lambda: bkv.bkv_fps_full(shape, h, m, k, picks, ws_full), reps)
        # the start and every pick stream the history once; norms and running maxima add 24 B per row per pick
        nbytes = (k + 1) * heads * m * d * es + k * heads * m * 24
        naive[m] = {"ms": ms, "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e6)}
        del h
    naive_beacons = torch.gather(hist, 2, picks.long().unsqueeze(-1).expand(N, Hq, k, d))
    xs = np.array(sorted(naive), dtype=np.float64)
    ys = np.array([naive[m]["ms"] for m in sorted(naive)])
    slope, icpt = np.polyfit(xs, ys, 1)
    naive_total = float(sum(icpt + slope * T * e for e in range(1, events + 1)))

    # continual: each period's queries go through the C-row buffer, then the beacon FPS, at every eviction
    eshape = bkv.make_shape(N, w.n_kv_heads, Hq, d, 1, hist.dtype)
    ws = bkv.alloc_workspace(eshape, w.n_recent, k, device=dev)
    qbuf = torch.empty(N, Hq, C, d, dtype=hist.dtype, device=dev)
    qcount = torch.zeros(N, Hq, dtype=torch.int32, device=dev)

    def continual():
        qcount.zero_()
        for blk in blocks:
            bkv.bkv_fps_update(eshape, blk, T, qbuf, qcount, C, M, ws)
            bkv.bkv_beacon_picks(eshape, qbuf, qcount, C, w.n_recent, k, ws)

    cont_total = timed(continual, reps)
    assert bkv.bkv_read_device_status(ws) == 0
    cont_beacons = bkv.ws_views(eshape, w.n_recent, k, ws)["beacon_rows"].clone()

    r_naive = covering_radius_deg(hist, naive_beacons)
    r_cont = covering_radius_deg(hist, cont_beacons)
    result = {
        "metric": "full-history FPS vs Continual FPS: time, memory, covering radius",
        "workload": "one layer of qwen3-14b-40layers-b32: %d query heads, a %d-step generation with an eviction every "
                    "%d steps, %d beacons; Continual FPS buffer %d -> %d" % (heads, n, T, k, C, M),
        "data": "synthetic",
        "dtype": "bf16 storage; FPS cosines in binary64 (full history) / fp32 with binary64 decisions (buffer)",
        "naive_per_eviction": {str(m): v for m, v in naive.items()},
        "naive_fit_ms": {"intercept": float(icpt), "per_query": float(slope)},
        "naive_generation_ms": naive_total,
        "naive_memory_bytes_per_head_at_end": n * d * es,
        "continual_generation_ms": cont_total,
        "continual_per_eviction_ms": cont_total / events,
        "continual_memory_bytes_per_head": C * d * es,
        "memory_ratio_at_end": (n * d * es) / (C * d * es),
        "generation_time_ratio": naive_total / cont_total,
        "covering_radius_deg_at_end": {
            "naive_mean": float(r_naive.mean()), "naive_max": float(r_naive.max()),
            "continual_mean": float(r_cont.mean()), "continual_max": float(r_cont.max()),
            "continual_over_naive_mean": float((r_cont / r_naive).mean()),
        },
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


def decode_compare(reps: int = 20):
    """One decode step of attention over the benchmark workload's cache, with
    and without the recent-query capture, and the eviction scoring it
    shortens: recent and beacon rows at eviction time, against the beacons
    alone raised to the captured maxima.  Prints its own JSON line."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bkv.load()
    w = configs.get(CFG)
    st = State(w, dev, n_pool=w.warm_steps // w.interval + 2)
    N, Hkv, Hq, d, L = st.N, w.n_kv_heads, w.n_q_heads, w.head_dim, w.length
    q = st.recent[st.block(0)][:, :, -1].contiguous()  # one query per head: [N, Hq, d]
    out = torch.empty(N, Hq, d, device=dev)
    capture = torch.zeros(N, Hkv, w.max_len, device=dev)
    ws_dec = torch.zeros(bkv.bkv_decode_workspace_size(st.shape), dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    plain = timed(lambda: bkv.bkv_decode_attention(st.shape, q, st.K, st.V, st.length, out, None, ws_dec))
    capt = timed(lambda: bkv.bkv_decode_attention(st.shape, q, st.K, st.V, st.length, out, capture, ws_dec))
    assert bkv.bkv_read_device_status(ws_dec) == 0
    kv_bytes = 2 * N * Hkv * L * d * st.K.element_size()
    # eviction scoring: recent + beacon rows at eviction time, or the beacons alone plus the capture
    bkv.bkv_beacon_picks(st.shape, st.qbuf, st.qcount, w.capacity, w.n_recent, w.n_beacons, st.ws)
    full = timed(lambda: st.score_picked(0, Group(st, 0, N, st.ws, None, None), torch.cuda.current_stream()))
    ws0 = bkv.alloc_workspace(st.shape, 0, w.n_beacons, device=dev)
    bkv.bkv_beacon_picks(st.shape, st.qbuf, st.qcount, w.capacity, 0, w.n_beacons, ws0)
    pos_now = st.pos_now[0]
    beac = timed(lambda: bkv.bkv_score_picked_capture(st.shape, st.K, st.length, capture, w.n_beacons, pos_now,
                                                      w.rope_theta, st.scores, ws0))
    assert bkv.bkv_read_device_status(ws0) == 0 and bkv.bkv_read_device_status(st.ws) == 0
    result = {
        "metric": "decode attention step with the recent-query capture; eviction scoring with and without it",
        "workload": "%s: %d slots x %d KV heads, %d query heads, cache %d, one query per head" % (w.name, N, Hkv, Hq, L),
        "data": "synthetic",
        "dtype": "bf16 storage, fp32 arithmetic",
        "decode_ms": plain,
        "decode_with_capture_ms": capt,
        "capture_overhead": capt / plain - 1.0,
        "decode_kv_GBps": kv_bytes / (plain * 1e6),
        "decode_with_capture_kv_GBps": kv_bytes / (capt * 1e6),
        "eviction_score_recent_and_beacons_ms": full,
        "eviction_score_beacons_plus_capture_ms": beac,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


def planted_recall(planted, kept, L, W):
    """(planted keys kept, planted keys among the candidates) of one eviction
    of one (slot, KV head): candidates are the rows [0, L - W) that the
    window does not protect; planted is a bool array over the L rows before
    the eviction, kept the ascending kept rows."""
    cand = int(np.count_nonzero(planted[:max(L - W, 0)]))
    kept = np.asarray(kept)
    k = kept[(kept >= 0) & (kept < L - W)]
    return int(np.count_nonzero(planted[k])), cand


POLICIES = ("beaconkv", "no_beacons", "mean", "initial_recent", "random")


def policy_recall(n_periods: int = 8, budget: int = 256, n_slots: int = 16, seed: int = 7, split_reps: int = 20):
    """Synthetic planted-key recall of the scoring policies the pages compare
    (BeaconKV's FPS beacons with max aggregation; no beacons, recent queries
    only; mean aggregation; InitialRecent; random representatives drawn from
    the buffer) and of the split between recent queries and beacons, on two
    data recipes of the one-layer Qwen3-4B workload: the preset as stated
    (5 % of keys planted along unit cluster centres, 10 % of queries around
    them, local queries i.i.d.), and the "revisit" recipe (local queries that
    resemble one another, clustered queries of the same norm that alone single
    out the planted keys).  Evicts to `budget` every period.  Also times the
    score stage against the split at 32 rows per query head on the benchmark
    workload.  Prints its own JSON line."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bkv.load()

    def study(w):
        N, Hkv, Hq, d = n_slots, w.n_kv_heads, w.n_q_heads, w.head_dim
        C, M, T, W, B = w.capacity, w.shrink_to, w.interval, w.window, budget
        L0 = Lmax = w.length  # the cache when the first eviction runs (2176)
        syn = synth.Synth(w, n_slots=N, seed=seed, device=dev)
        shape = bkv.make_shape(N, Hkv, Hq, d, Lmax, torch.bfloat16)
        n_warm = w.warm_steps // T
        warm = [syn.query_block(b) for b in range(n_warm)]
        K0, V0, P0 = syn.keys(max_len=Lmax), syn.values(max_len=Lmax), syn.planted(max_len=Lmax)
        blocks = [syn.query_block(n_warm + p) for p in range(n_periods)]
        newk = [syn.keys(max_len=T, block=1 + p) for p in range(n_periods)]
        newv = [syn.values(max_len=T, block=1 + p) for p in range(n_periods)]
        newp = [syn.planted(max_len=T, block=1 + p) for p in range(n_periods)]
        qbuf0 = torch.zeros(N, Hq, C, d, dtype=torch.bfloat16, device=dev)
        qcount0 = torch.zeros(N, Hq, dtype=torch.int32, device=dev)
        ws0 = bkv.alloc_workspace(shape, 0, 0, device=dev)
        for blk in warm:
            bkv.bkv_fps_update(shape, blk, T, qbuf0, qcount0, C, M, ws0)
        torch.cuda.synchronize()
        gen = torch.Generator(device=dev)

        def run(policy, R, nb):
            first_q = warm[0][:, :, :nb].contiguous()  # InitialRecent: each head's earliest queries
            K, V, planted = K0.clone(), V0.clone(), P0.clone()
            qbuf, qcount = qbuf0.clone(), qcount0.clone()
            length = torch.full((N,), L0, dtype=torch.int32, device=dev)
            ws = bkv.alloc_workspace(shape, R, nb, device=dev)
            scores = torch.zeros(N, Hkv, Lmax, device=dev)
            kept = torch.empty(N, Hkv, B, dtype=torch.int32, device=dev)
            gen.manual_seed(seed)
            kept_planted = cand_planted = 0
            per_eviction = []
            for p in range(n_periods):
                blk = blocks[p]
                bkv.bkv_fps_update(shape, blk, T, qbuf, qcount, C, M, ws)
                now = (n_warm + p + 1) * T - 1
                rpos = torch.arange(now - R + 1, now + 1, dtype=torch.int32, device=dev).repeat(N, 1).contiguous()
                pos_now = torch.full((N,), now, dtype=torch.int32, device=dev)
                recent = blk[:, :, T - R:].contiguous()
                agg = bkv.AGG_MEAN if policy == "mean" else bkv.AGG_MAX
                if policy in ("beaconkv", "mean"):
                    bkv.bkv_beacon_picks(shape, qbuf, qcount, C, R, nb, ws)
                elif policy == "no_beacons":
                    bkv.bkv_beacon_rows(shape, None, 0, None, R, 0, ws)
                elif policy == "initial_recent":
                    idx = torch.arange(nb, dtype=torch.int32, device=dev).repeat(N, Hq, 1).contiguous()
                    bkv.bkv_beacon_rows(shape, first_q, nb, idx, R, nb, ws)
                else:  # nb distinct live rows of each head's buffer, drawn at random
                    r = torch.rand(N, Hq, C, generator=gen, device=dev)
                    r = torch.where(torch.arange(C, device=dev) < qcount.unsqueeze(-1), r, torch.full_like(r, 2.0))
                    idx = r.argsort(dim=-1)[:, :, :nb].to(torch.int32)
                    idx = torch.where(torch.arange(nb, device=dev) < qcount.unsqueeze(-1), idx,
                                      torch.full_like(idx, -1))
                    bkv.bkv_beacon_rows(shape, qbuf, C, idx.contiguous(), R, nb, ws)
                bkv.bkv_score_picked_agg(shape, K, length, recent, rpos, R, nb, pos_now, w.rope_theta, agg, scores, ws)
                L = int(length[0])
                bkv.bkv_select_compact(shape, scores, K, V, length, B, W, kept, ws)
                pl = planted.cpu().numpy()
                kp = kept.cpu().numpy()
                k_sum = c_sum = 0
                for n in range(N):
                    for h in range(Hkv):
                        a_, b_ = planted_recall(pl[n, h], kp[n, h], L, W)
                        k_sum, c_sum = k_sum + a_, c_sum + b_
                per_eviction.append(k_sum / max(c_sum, 1))
                kept_planted, cand_planted = kept_planted + k_sum, cand_planted + c_sum
                # the planted flags follow their rows; the period's new tokens are appended after the budget
                planted[:, :, :B] = torch.gather(planted, 2, kept.long())
                planted[:, :, B:] = False
                K[:, :, B:B + T].copy_(newk[p])
                V[:, :, B:B + T].copy_(newv[p])
                planted[:, :, B:B + T] = newp[p]
                length.fill_(B + T)
            torch.cuda.synchronize()
            assert bkv.bkv_read_device_status(ws) == 0
            return {"recall": kept_planted / max(cand_planted, 1),
                    "recall_per_eviction": per_eviction,
                    "planted_fraction_of_cache_at_end": float(planted[:, :, :B].float().mean().item())}

        R, nb = w.n_recent, w.n_beacons
        out = {"policies": {pname: run(pname, R, 0 if pname == "no_beacons" else nb)
                            for pname in POLICIES},
               "split": [dict(recent=r_, beacons=b_, **run("beaconkv", r_, b_))
                         for r_, b_ in ((32, 0), (24, 8), (16, 16), (8, 24), (1, 31))],
               "workload": "%s x %d slots: 8 KV / 32 query heads, d=128, bf16, %.0f%% of keys planted along the %d "
                           "query-cluster centres, %.0f%% of queries around those centres (norm scale %.3g, noise "
                           "%.2g), local queries %s; first eviction %d -> %d, then %d periods of %d new tokens "
                           "evicted back to %d (window %d, buffer %d -> %d)"
                           % (w.name, N, 100 * w.plant_rate, w.n_centres, 100 * w.p_global, w.global_scale, w.sigma,
                              "i.i.d. N(0, I)" if w.local_scale == 0 else
                              "%.3g * a shared direction + N(0, I)" % w.local_scale,
                              L0, B, n_periods - 1, T, B, W, C, M),
               "planted_fraction_of_cache_at_start": float(P0.float().mean().item())}
        return out

    w2 = configs.get(2)
    recipes = {"stated": study(w2), "revisit": study(configs.revisit(w2))}

    # scoring time against the recent / beacon split at 32 rows per query head, benchmark workload
    w3 = configs.get(CFG)
    st = State(w3, dev, n_pool=w3.warm_steps // w3.interval + 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(split_reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / split_reps

    split = []
    blk = st.blocks[st.block(0)]
    now = int(st.pos_now[0, 0])
    for r_, b_ in ((32, 0), (24, 8), (16, 16), (8, 24), (1, 31)):
        ws = bkv.alloc_workspace(st.shape, r_, b_, device=dev)
        rec = blk[:, :, -r_:].contiguous()
        rp = torch.arange(now - r_ + 1, now + 1, dtype=torch.int32, device=dev).repeat(st.N, 1).contiguous()
        picks_ms = timed(lambda: bkv.bkv_beacon_picks(st.shape, st.qbuf, st.qcount, w3.capacity, r_, b_, ws))
        score_ms = timed(lambda: bkv.bkv_score_picked(st.shape, st.K, st.length, rec, rp, r_, b_, st.pos_now[0],
                                                      w3.rope_theta, st.scores, ws))
        assert bkv.bkv_read_device_status(ws) == 0
        split.append({"recent": r_, "beacons": b_, "beacon_fps_ms": picks_ms, "score_ms": score_ms})
        del ws

    result = {
        "metric": "planted-key recall of the scoring policies and of the recent/beacon split; scoring time against "
                  "the split",
        "data": "synthetic",
        "recall_definition": "planted keys kept / planted keys among the eviction candidates (rows outside the "
                             "window), summed over evictions and (slot, KV head) units",
        "recipes": recipes,
        "split_timing_workload": w3.name + " (4,608 units, cache 2176, 32 observation rows per query head)",
        "split_timing": split,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(result), flush=True)


def load_traffic(src_hash, workload):
    """The recorded counter figures, if they were taken on this workload with
    these kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except Exception:
        return None
    if t.get("kernel_source_hash") != src_hash or t.get("workload") != workload:
        return None
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--no-hole-fill", action="store_true", help="skip the hole-filling layout phase")
    ap.add_argument("--no-overlap", action="store_true", help="skip the overlapped and pipelined schedules")
    ap.add_argument("--groups", type=int, default=3, help="slot groups of the pipelined schedule")
    ap.add_argument("--picks-after-scoring", action="store_true",
                    help="order-preserving overlapped and pipelined schedules: start the beacon FPS of pass i+1 when "
                         "pass i's scoring ends (default: when its compaction ends)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time for the CPU baseline")
    ap.add_argument("--no-all-cores", action="store_true", help="skip the all-host-threads oracle timing")
    ap.add_argument("--workload", type=int, default=CFG, choices=(3, 4, 5),
                    help="3: Qwen3-4B b16 B=2K (default); 4: Qwen3-4B b320 B=1K; 5: Qwen3-14B b32 B=4K")
    ap.add_argument("--decode-compare", action="store_true",
                    help="instead of the eviction pass: decode attention with and without the recent-query capture")
    ap.add_argument("--fps-compare", action="store_true",
                    help="instead of the eviction pass: full-history FPS vs Continual FPS on one Qwen3-14B layer")
    ap.add_argument("--policy-recall", action="store_true",
                    help="instead of the eviction pass: planted-key recall of the scoring policies and the scoring "
                         "time of the recent/beacon split")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.fps_compare:
        fps_compare()
        return
    if args.policy_recall:
        policy_recall()
        return
    if args.decode_compare:
        decode_compare()
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = configs.get(args.workload)
    bkv.load()

    block_bytes = w.n_slots * w.n_q_heads * w.interval * w.head_dim * (2 if w.dtype == "bf16" else 4)
    # one block per pass of a phase (warm-up passes, timed passes, and the primed next one)
    n_pool = min(POOL_MAX, args.warmup + args.steps + 1, max(2, int(POOL_BYTES // block_bytes)))
    st = State(w, dev, n_pool=n_pool)
    if not args.no_cpu_baseline:
        # pristine copies of the cache for the oracle sample, taken before any compaction
        st.K_pristine = st.K.clone()
        st.V_pristine = st.V.clone()
    cp = copy_probe(dev)
    log("copy probe: %.0f GB/s" % cp["GBps"])

    def grow(i, g):
        st.length[g.sl].copy_(st.len_full[g.sl])
        st.append_new_tokens(i, g)

    def tail(i, rec, g):
        rec("select", 0)
        bkv.bkv_select(g.shape, st.scores[g.sl], st.length[g.sl], w.budget, w.window, st.kept[g.sl], g.ws)
        rec("select", 1)
        rec("compact", 0)
        bkv.bkv_compact(g.shape, st.K[g.sl], st.V[g.sl], st.length[g.sl], w.budget, st.kept[g.sl], g.ws)
        rec("compact", 1)

    K = args.steps
    # serial schedule first: every kernel runs alone, so its events time it cleanly (stage times, roofline)
    elapsed, stage_ms, stage_spread, rows_moved = timed_passes(Schedule(st, grow, tail, False), args.warmup, K)
    serial = {"passes_per_s": K / elapsed, "ms_per_step": elapsed * 1e3 / K}
    overlapped = pipelined = None
    if not args.no_overlap:
        log("timing the overlapped schedule")
        el, sm, sp, _ = timed_passes(Schedule(st, grow, tail, True, picks_after_tail=not args.picks_after_scoring),
                                     args.warmup, K)
        overlapped = {
            "schedule": "the ingest of pass i+1 runs on a second stream (default priority) while pass i scores, and "
                        "its beacon FPS once pass i has compacted (beside pass i+1's new-token append; with "
                        "--picks-after-scoring once pass i has scored); same work per pass",
            "passes_per_s": K / el,
            "ms_per_step": el * 1e3 / K,
            "stage_ms": sm,
            "stage_ms_p10_p50_p90": sp,
        }
        log("timing the pipelined schedule (%d slot groups)" % args.groups)
        el, sm, sp, _ = timed_passes(Schedule(st, grow, tail, True, groups=args.groups,
                                              picks_after_tail=not args.picks_after_scoring), args.warmup, K)
        pipelined = {
            "schedule": "the slots split into %d groups, each with its own streams and workspace; the groups' scorings "
                        "take turns, so one group selects and compacts while the next one scores; ingest and beacon "
                        "FPS of pass i+1 on the side stream as above; same work per pass; stage times of group 0"
                        % args.groups,
            "groups": args.groups,
            "passes_per_s": K / el,
            "ms_per_step": el * 1e3 / K,
            "stage_ms": sm,
            "stage_ms_p10_p50_p90": sp,
        }
    head = pipelined or serial
    ms_per_step = head["ms_per_step"]
    passes_per_s = head["passes_per_s"]

    # algorithmic bytes
    units = st.N * w.n_kv_heads
    row_bytes = w.head_dim * 2
    L = w.length
    score_bytes = units * (L * row_bytes + w.obs_rows * row_bytes + L * 4)
    compact_bytes = (rows_moved / K) * row_bytes * 2          # rows_moved counts K and V rows
    entries = units * L
    score_compact_gbps = (score_bytes + compact_bytes) / ((stage_ms["score"] + stage_ms["compact"]) * 1e6)

    # the benchmark spec's figure: score + compaction of a pass, algorithmic bytes
    # over the two stages' time, each kernel alone (serial schedule)
    pass_bytes = score_bytes + compact_bytes
    pass_ms = stage_ms["score"] + stage_ms["compact"]
    north = {
        "what": "score + order-preserving compaction of one eviction pass: algorithmic bytes / HIP-event time of the "
                "two stages (serial schedule, each running alone; the score stage is the RoPE table and score "
                "kernels, the beacon FPS is timed as its own stage)",
        "algorithmic_bytes": pass_bytes,
        "ms": pass_ms,
        "GBps": pass_bytes / (pass_ms * 1e6),
        "frac_of_peak": pass_bytes / (pass_ms * 1e6) / HBM_PEAK_GBPS,
        "target_frac": NORTH_STAR_FRAC,
        "meets_target": pass_bytes / (pass_ms * 1e6) / HBM_PEAK_GBPS >= NORTH_STAR_FRAC,
        "whole_pass": {
            "what": "the same bytes over the reported (pipelined, else serial) wall-clock time of a whole pass, "
                    "which also holds the new tokens, the ingest and the beacon FPS",
            "ms_per_pass": ms_per_step,
            "GBps": pass_bytes / (ms_per_step * 1e6),
            "frac_of_peak": pass_bytes / (ms_per_step * 1e6) / HBM_PEAK_GBPS,
        },
    }

    dominant = max(("score", "compact"), key=lambda n: stage_ms[n])
    dom_bytes = compact_bytes if dominant == "compact" else score_bytes
    achieved = dom_bytes / (stage_ms[dominant] * 1e6)
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash, w.name)
    dom_traffic = None
    if traffic and dominant in traffic.get("kernels", {}):
        dom_traffic = traffic["kernels"][dominant].get("hbm_bytes_per_launch")
    if traffic and all(k in traffic.get("kernels", {}) for k in ("score", "compact")):
        north["traffic"] = sum(traffic["kernels"][k]["hbm_bytes_per_launch"] for k in ("score", "compact"))
    else:
        north["traffic"] = None
    score_traffic = (traffic["kernels"]["score"]["hbm_bytes_per_launch"]
                     if traffic and "score" in traffic.get("kernels", {}) else None)

    result = {
        "metric": ("eviction passes/s + KV entries scored/s (HBM GB/s, % peak), Qwen3-4B b16 B=2K"
                   if args.workload == CFG else "eviction passes/s + KV entries scored/s, %s" % w.name),
        "value": passes_per_s,
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "batch": w.batch, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "cache_len": L, "budget": w.budget,
                   "window": w.window, "recent": w.n_recent, "beacons": w.n_beacons, "fps_capacity": w.capacity,
                   "fps_shrink_to": w.shrink_to, "queries_per_step": w.interval},
        "entries_scored_per_s": entries * passes_per_s,
        "score_compact_GBps": score_compact_gbps,
        "score_compact_frac_of_peak": score_compact_gbps / HBM_PEAK_GBPS,
        "north_star_pass": north,
        "score_kernel_roofline": {
            "kernel": "score", "bound": "hbm", "achieved": score_bytes / (stage_ms["score"] * 1e6),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": score_bytes / (stage_ms["score"] * 1e6) / HBM_PEAK_GBPS, "traffic": score_traffic,
        },
        "schedule": ("pipelined (see 'pipelined'); stage_ms and the roofline come from the serial schedule, where "
                     "every kernel runs alone" if pipelined else "serial: every stage on one stream"),
        "serial": serial,
        "stage_ms": stage_ms,
        "stage_ms_p10_p50_p90": stage_spread,
        "algorithmic_bytes_per_step": {"score": score_bytes, "compact": compact_bytes},
        "copy_probe_GBps": cp["GBps"],
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": dom_traffic,
        },
        "kernel_source_hash": src_hash,
    }
    if overlapped:
        result["overlapped"] = overlapped
        result["pipelined"] = pipelined
    if not args.no_hole_fill:
        log("timing the hole-filling layout on the same workload")
        result["hole_fill"] = time_hole_fill(st, args.warmup, K, False)
        if not args.no_overlap:
            for name, groups in (("overlapped", 1), ("pipelined", args.groups)):
                ov = time_hole_fill(st, args.warmup, K, True, groups=groups)
                result["hole_fill"][name] = {"passes_per_s": ov["passes_per_s"], "ms_per_step": ov["ms_per_step"],
                                             "stage_ms": ov["stage_ms"],
                                             "stage_ms_p10_p50_p90": ov["stage_ms_p10_p50_p90"]}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        sample = OracleSample(st)
        result["cpu_baseline"] = cpu_baseline(sample, budget_s=args.cpu_budget)
        if not args.no_all_cores:
            log("timing the CPU oracle on %d host threads" % host_threads())
            result["cpu_baseline_all_cores"] = cpu_baseline_all_cores(sample, budget_s=args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
