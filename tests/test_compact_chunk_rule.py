"""The hazard rule of the chunked order-preserving compaction, checked on the
CPU against brute force.  Destinations [f, cnt) of a (unit, tensor) are cut
into chunks of CR rows by absolute row; chunk j moves rows kept[i] -> i for
i in [jCR, (j+1)CR) within [f, cnt), reading all its sources before writing
any destination.  The kernel lets chunk j write after waiting only for the
earlier chunks found by walking back from j - 1 while the earlier chunk moves
rows and its last source kept[(j'+1)CR - 1] lies at or beyond j's first moved
row.  Brute force: every chunk whose source set meets chunk j's destination
set must finish its reads before j writes.  The rule must name every earlier
such chunk, and no later chunk may read a row that j writes."""
import numpy as np
import pytest


def chunk_ranges(f, cnt, CR, nchunk):
    out = []
    for j in range(nchunk):
        s, e = max(f, j * CR), min(cnt, (j + 1) * CR)
        out.append((s, e) if s < e else None)
    return out


def rule_waits(kept, f, cnt, CR, j, start):
    """Chunks the kernel waits for before chunk j writes."""
    waits = []
    jp = j - 1
    while jp >= 0:
        last = (jp + 1) * CR - 1
        if last < f or kept[last] < start:
            break
        waits.append(jp)
        jp -= 1
    return waits


def random_kept(gen, L, B, kind):
    if kind == "random":
        return np.sort(gen.choice(L, size=B, replace=False))
    if kind == "front":
        return np.arange(L - B, L)
    if kind == "runs":  # one evicted run (up to every evicted row), the rest of the holes at random
        holes = L - B
        keep = np.ones(L, bool)
        run = int(gen.integers(0, holes + 1))
        at = int(gen.integers(0, L - run + 1))
        keep[at:at + run] = False
        if holes > run:
            keep[gen.choice(np.flatnonzero(keep), size=holes - run, replace=False)] = False
        return np.flatnonzero(keep)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["random", "front", "runs"])
@pytest.mark.parametrize("CR", [4, 16, 64])
def test_the_wait_rule_covers_every_hazard(kind, CR):
    gen = np.random.default_rng(CR * 7 + len(kind))
    for trial in range(300):
        L = int(gen.integers(2, 400))
        B = int(gen.integers(1, L + 1))
        kept = random_kept(gen, L, B, kind)
        assert len(kept) == B and np.all(np.diff(kept) > 0)
        cnt = B
        ident = np.arange(cnt)
        f = cnt if np.array_equal(kept, ident) else int(np.argmax(kept != ident))
        nchunk = (L + CR - 1) // CR
        ranges = chunk_ranges(f, cnt, CR, nchunk)
        reads = [set(kept[r[0]:r[1]].tolist()) if r else set() for r in ranges]
        writes = [set(range(r[0], r[1])) if r else set() for r in ranges]
        for j, r in enumerate(ranges):
            if r is None:
                continue
            start = r[0]
            must = {jp for jp in range(j) if reads[jp] & writes[j]}
            got = set(rule_waits(kept, f, cnt, CR, j, start))
            assert must <= got, (L, B, CR, j, sorted(must - got))
            # every chunk in the wait set moves rows (its flag will be set)
            assert all(ranges[jp] is not None for jp in got)
            # a later chunk never reads a row chunk j writes
            assert not any(reads[jl] & writes[j] for jl in range(j + 1, nchunk))


def test_the_chunked_moves_equal_a_gather_in_any_order_the_rule_allows():
    """Replaying the moves chunk by chunk in a random order that respects the
    waits (each chunk reads all its rows, then writes once its waits are
    done) always leaves row i = old row kept[i]."""
    gen = np.random.default_rng(3)
    for trial in range(200):
        L = int(gen.integers(2, 300))
        B = int(gen.integers(1, L + 1))
        CR = int(gen.choice([3, 8, 32]))
        kept = np.sort(gen.choice(L, size=B, replace=False))
        cnt = B
        ident = np.arange(cnt)
        f = cnt if np.array_equal(kept, ident) else int(np.argmax(kept != ident))
        nchunk = (L + CR - 1) // CR
        ranges = chunk_ranges(f, cnt, CR, nchunk)
        rows = np.arange(L) * 10 + 7  # row contents
        want = rows.copy()
        want[:cnt] = rows[kept]
        state = {j: "todo" for j, r in enumerate(ranges) if r is not None}
        data = {}
        while any(v != "done" for v in state.values()):
            j = int(gen.choice([k for k, v in state.items() if v != "done"]))
            s, e = ranges[j]
            if state[j] == "todo":  # read all sources
                data[j] = rows[kept[s:e]].copy()
                state[j] = "read"
            elif all(state[jp] in ("read", "done") for jp in rule_waits(kept, f, cnt, CR, j, s)):
                rows[s:e] = data[j]
                state[j] = "done"
        assert np.array_equal(rows, want), (L, B, CR)
