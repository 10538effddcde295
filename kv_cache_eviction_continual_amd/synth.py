"""Seeded synthetic inputs for the eviction hot path.

This module only draws random numbers and lays them out; it performs none of
the method's arithmetic (no normalisation for similarity, no rotary
embedding, no attention, no selection).  Tests, the benchmark and the smoke
check use it to feed the same inputs to the HIP library and to the CPU
oracle.

Workload structure (a stand-in for the long reasoning traces the pages
measure on, which need model weights and benchmark datasets):
  * a query at decode step t has position t;
  * each query head draws a fraction ``p_global`` of its queries around one
    of ``n_centres`` cluster centres (centre + sigma * N(0, I)) and the rest
    i.i.d. N(0, I); the centres belong to the (slot, KV head) and are shared
    by the query heads of its group.  This mirrors the observation that
    global, revisiting queries form a few tight clusters in query space
    (wzjinhao.cn news article 56682, section "藏在混乱背后的秩序");
  * cached keys (stored post-RoPE) and values are i.i.d. N(0, 1); a fraction
    ``plant_rate`` of keys is planted at sqrt(d) * centre + 0.1 * N(0, I);
  * storage rounding to bfloat16 is torch's round-to-nearest-even cast.

Draws use one torch generator per (workload, seed, stream, block) so that a
block can be regenerated on its own.  Tensors are generated on the requested
device; the oracle receives host copies of the very same values.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

_STREAM_CENTRES = 1
_STREAM_QUERY = 2
_STREAM_KEYS = 3
_STREAM_VALUES = 4
_STREAM_SCORES = 5
_STREAM_MISC = 6


def _seed(*key: int) -> int:
    state = np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key]).generate_state(2, dtype=np.uint64)
    return int(state[0] >> np.uint64(1))


def generator(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


def storage_dtype(w_or_name) -> torch.dtype:
    name = w_or_name.dtype if isinstance(w_or_name, Workload) else w_or_name
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def to_storage(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Cast float32 draws to the storage type (round to nearest even)."""
    return x.to(storage_dtype(dtype)).contiguous()


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """Host copy of a storage tensor: float32, or uint16 bfloat16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def from_numpy_storage(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    if a.dtype == np.float32:
        return torch.from_numpy(a.copy()).to(device)
    raise TypeError(a.dtype)


class Synth:
    """Seeded input source for one workload over ``n_slots`` sequence slots."""

    def __init__(self, w: Workload, n_slots: int | None = None, seed: int = 0, device="cpu", tag: int = 0):
        self.w = w
        self.N = int(n_slots if n_slots is not None else w.n_slots)
        self.seed = int(seed)
        self.tag = int(tag)
        self.device = torch.device(device)
        g = generator(self.device, self.tag, self.seed, _STREAM_CENTRES)
        c = torch.randn(self.N, w.n_kv_heads, w.n_centres, w.head_dim, generator=g, device=self.device)
        if w.centre_kind == "unit":
            c = c / c.norm(dim=-1, keepdim=True)
        self.centres = c
        self.local_dir = None
        if w.local_scale > 0:  # one unit direction per (slot, KV head) shared by its local queries
            gl = generator(self.device, self.tag, self.seed, _STREAM_CENTRES, 1)
            u = torch.randn(self.N, w.n_kv_heads, w.head_dim, generator=gl, device=self.device)
            self.local_dir = u / u.norm(dim=-1, keepdim=True)

    # -- queries --------------------------------------------------------------
    def query_block(self, block: int, steps: int | None = None) -> torch.Tensor:
        """Pre-RoPE queries of decode steps [block*interval, block*interval+steps):
        storage tensor [N, Hq, steps, d]."""
        w = self.w
        steps = w.interval if steps is None else steps
        g = generator(self.device, self.tag, self.seed, _STREAM_QUERY, block)
        N, Hq, d = self.N, w.n_q_heads, w.head_dim
        z = torch.randn(N, Hq, steps, d, generator=g, device=self.device)
        u = torch.rand(N, Hq, steps, generator=g, device=self.device)
        m = torch.randint(0, w.n_centres, (N, Hq, steps), generator=g, device=self.device)
        cq = self.centres.repeat_interleave(w.group, dim=1)  # [N, Hq, n_centres, d]
        cen = torch.gather(cq, 2, m.unsqueeze(-1).expand(N, Hq, steps, d))
        local = z
        if self.local_dir is not None:
            local = z + w.local_scale * self.local_dir.repeat_interleave(w.group, dim=1).unsqueeze(2)
        glob = cen + w.sigma * z if w.global_scale == 1.0 else w.global_scale * cen + w.sigma * z
        q = torch.where((u < w.p_global).unsqueeze(-1), glob, local)
        return to_storage(q, w.dtype)

    def stream(self, steps: int) -> torch.Tensor:
        """The first ``steps`` queries of every head, block by block: [N, Hq, steps, d]."""
        w = self.w
        blocks = []
        done = 0
        b = 0
        while done < steps:
            take = min(w.interval, steps - done)
            blk = self.query_block(b)
            blocks.append(blk[:, :, :take])
            done += take
            b += 1
        return torch.cat(blocks, dim=2).contiguous()

    # -- cache ----------------------------------------------------------------
    def keys(self, max_len: int | None = None, block: int = 0) -> torch.Tensor:
        w = self.w
        Lm = w.max_len if max_len is None else max_len
        g = generator(self.device, self.tag, self.seed, _STREAM_KEYS, block)
        N, H, d = self.N, w.n_kv_heads, w.head_dim
        z = torch.randn(N, H, Lm, d, generator=g, device=self.device)
        if w.plant_rate > 0:
            u = torch.rand(N, H, Lm, generator=g, device=self.device)
            m = torch.randint(0, w.n_centres, (N, H, Lm), generator=g, device=self.device)
            cen = torch.gather(self.centres, 2, m.unsqueeze(-1).expand(N, H, Lm, d))
            z = torch.where((u < w.plant_rate).unsqueeze(-1), (d ** 0.5) * cen + 0.1 * z, z)
        return to_storage(z, w.dtype)

    def planted(self, max_len: int | None = None, block: int = 0) -> torch.Tensor:
        """Which rows of keys(max_len, block) are planted near a centre: the
        same draws replayed, bool [N, Hkv, Lm] (all False without planting)."""
        w = self.w
        Lm = w.max_len if max_len is None else max_len
        N, H, d = self.N, w.n_kv_heads, w.head_dim
        if w.plant_rate <= 0:
            return torch.zeros(N, H, Lm, dtype=torch.bool, device=self.device)
        g = generator(self.device, self.tag, self.seed, _STREAM_KEYS, block)
        torch.randn(N, H, Lm, d, generator=g, device=self.device)
        u = torch.rand(N, H, Lm, generator=g, device=self.device)
        return u < w.plant_rate

    def values(self, max_len: int | None = None, block: int = 0) -> torch.Tensor:
        w = self.w
        Lm = w.max_len if max_len is None else max_len
        g = generator(self.device, self.tag, self.seed, _STREAM_VALUES, block)
        z = torch.randn(self.N, w.n_kv_heads, Lm, w.head_dim, generator=g, device=self.device)
        return to_storage(z, w.dtype)

    # -- misc -----------------------------------------------------------------
    def scores(self, L: int, tie_fraction: float = 0.0, block: int = 0) -> torch.Tensor:
        """Positive float32 scores [N, Hkv, L]; optionally a fraction of entries
        copied from a few shared values to create exact ties."""
        w = self.w
        g = generator(self.device, self.tag, self.seed, _STREAM_SCORES, block)
        s = torch.rand(self.N, w.n_kv_heads, L, generator=g, device=self.device) * 1e-3 + 1e-6
        if tie_fraction > 0:
            u = torch.rand(self.N, w.n_kv_heads, L, generator=g, device=self.device)
            pool = torch.rand(4, generator=g, device=self.device) * 1e-3 + 1e-6
            pick = torch.randint(0, 4, (self.N, w.n_kv_heads, L), generator=g, device=self.device)
            s = torch.where(u < tie_fraction, pool[pick], s)
        return s.contiguous()

    def randint(self, lo: int, hi: int, shape, block: int = 0) -> torch.Tensor:
        g = generator(self.device, self.tag, self.seed, _STREAM_MISC, block)
        return torch.randint(lo, hi, tuple(shape), generator=g, device=self.device, dtype=torch.int64)

    def randn(self, shape, block: int = 0) -> torch.Tensor:
        g = generator(self.device, self.tag, self.seed, _STREAM_MISC, 1000 + block)
        return torch.randn(*shape, generator=g, device=self.device)


def recent_positions(n_slots: int, n_recent: int, now: int) -> np.ndarray:
    """Positions of the last ``n_recent`` decode steps ending at ``now``
    (negative positions mark queries that do not exist yet)."""
    base = np.arange(now - n_recent + 1, now + 1, dtype=np.int32)
    base[base < 0] = -1
    return np.broadcast_to(base, (n_slots, n_recent)).copy()
