"""Workload presets of the eviction hot path.

Each preset fixes the cache shape, the eviction budget and the beacon
parameters of one synthetic workload.  The defaults of 16 beacon queries, 16
recent queries and a 32-entry window follow aimodeling.com "BeaconKV: Beacon
Queries Fix KV Eviction for Long Reasoning", section "Beacon queries
anticipate what will be revisited".  Model shapes: Qwen3-4B is 36 layers, 32
query heads over 8 KV heads, head dim 128, RoPE base 1e6; Qwen3-14B is 40
layers, 40 query heads over 8 KV heads, head dim 128, RoPE base 1e6.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int          # model layers flattened into sequence slots
    batch: int           # sequences per layer
    n_kv_heads: int      # Hkv
    group: int           # G = query heads per KV head
    head_dim: int        # d
    dtype: str           # "f32" or "bf16" storage of K, V and queries
    rope_theta: float
    length: int          # L: cache length when eviction runs
    budget: int          # B_KV: entries kept (window included)
    window: int          # W: recent entries always kept
    n_recent: int        # R: recent observation queries per query head
    n_beacons: int       # nb: beacons per query head
    capacity: int        # C: Continual-FPS buffer capacity
    shrink_to: int       # M: FPS target size when the buffer fills
    interval: int        # decode steps between evictions
    # synthetic query / key distribution
    p_global: float      # fraction of queries drawn around a cluster centre
    n_centres: int
    centre_kind: str     # "gauss" (N(0, I) centres) or "unit" (unit-norm centres)
    sigma: float         # per-coordinate noise of clustered queries
    plant_rate: float    # fraction of keys planted near a centre
    warm_steps: int      # query-stream length used to reach a realistic buffer state
    # optional structure for the policy ablation (the defaults leave every
    # preset's draws unchanged): local queries are local_scale * u + N(0, I)
    # with one unit direction u per (slot, KV head), so that they resemble one
    # another; clustered queries are global_scale * centre + sigma * N(0, I)
    local_scale: float = 0.0
    global_scale: float = 1.0

    @property
    def n_slots(self) -> int:
        return self.layers * self.batch

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def max_len(self) -> int:
        return self.length

    @property
    def obs_rows(self) -> int:
        return self.group * (self.n_recent + self.n_beacons)


CONFIGS = {
    # 1. tiny single-head eviction, binary32
    1: Workload("tiny-1kv-gqa4-d64-f32", layers=1, batch=1, n_kv_heads=1, group=4, head_dim=64,
                dtype="f32", rope_theta=1e4, length=512, budget=128, window=16, n_recent=8,
                n_beacons=8, capacity=64, shrink_to=16, interval=128, p_global=0.15, n_centres=3,
                centre_kind="gauss", sigma=0.1, plant_rate=0.0, warm_steps=512),
    # 2. one layer at Qwen3-4B shape, cache 2176 evicted to 2048
    2: Workload("qwen3-4b-1layer-b1", layers=1, batch=1, n_kv_heads=8, group=4, head_dim=128,
                dtype="bf16", rope_theta=1e6, length=2176, budget=2048, window=32, n_recent=16,
                n_beacons=16, capacity=128, shrink_to=16, interval=128, p_global=0.10, n_centres=6,
                centre_kind="unit", sigma=0.1, plant_rate=0.05, warm_steps=2176),
    # 3. all 36 layers of Qwen3-4B at batch 16, B_KV = 2048, evict every 128 steps
    3: Workload("qwen3-4b-36layers-b16-B2048", layers=36, batch=16, n_kv_heads=8, group=4,
                head_dim=128, dtype="bf16", rope_theta=1e6, length=2176, budget=2048, window=32,
                n_recent=16, n_beacons=16, capacity=128, shrink_to=16, interval=128, p_global=0.15,
                n_centres=3, centre_kind="gauss", sigma=0.1, plant_rate=0.0, warm_steps=2176),
    # 4. Qwen3-4B at batch 320, B_KV = 1024
    4: Workload("qwen3-4b-36layers-b320-B1024", layers=36, batch=320, n_kv_heads=8, group=4,
                head_dim=128, dtype="bf16", rope_theta=1e6, length=1152, budget=1024, window=32,
                n_recent=16, n_beacons=16, capacity=128, shrink_to=16, interval=128, p_global=0.15,
                n_centres=3, centre_kind="gauss", sigma=0.1, plant_rate=0.0, warm_steps=1152),
    # 5. Qwen3-14B at batch 32, B_KV = 4096, buffer 256 -> 32, 32 beacons, 10 clusters
    5: Workload("qwen3-14b-40layers-b32-B4096", layers=40, batch=32, n_kv_heads=8, group=5,
                head_dim=128, dtype="bf16", rope_theta=1e6, length=4224, budget=4096, window=32,
                n_recent=16, n_beacons=32, capacity=256, shrink_to=32, interval=128, p_global=0.15,
                n_centres=10, centre_kind="gauss", sigma=0.1, plant_rate=0.0, warm_steps=4224),
}


def revisit(w: Workload) -> Workload:
    """The ablation's "revisit" recipe on top of a preset: local queries
    that resemble one another (a shared direction of norm sqrt(d), cosine
    about 0.5 between two of them) and clustered global queries of the same
    norm around unit centres (noise 0.3 per coordinate), which alone single
    out the keys planted along those centres."""
    d = w.head_dim
    return replace(w, name=w.name + "-revisit", centre_kind="unit", local_scale=d ** 0.5, global_scale=d ** 0.5,
                   sigma=0.3, plant_rate=w.plant_rate if w.plant_rate > 0 else 0.05)


def get(cfg: int, **overrides) -> Workload:
    w = CONFIGS[cfg]
    return replace(w, **overrides) if overrides else w
