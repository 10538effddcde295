"""CPU oracle of the BeaconKV eviction hot path (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle.so`` (plain C,
binary64 arithmetic, single-threaded; source ``bkv_oracle.c`` in this folder)
with NumPy marshalling and per-head loops.  It shares no code with the HIP
library.

Storage arrays are NumPy ``float32`` (binary32) or ``uint16`` (bfloat16 bit
patterns).  Every function says which step of the method it follows; the
citations are in ``bkv_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bkv_oracle.c")
# BKV_ORACLE_LIB names another build of the same source to load instead (the
# sanitizer test builds one with address and undefined-behaviour checks)
_LIB = os.environ.get("BKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1


BUILD_FLAGS = ("-O2", "-std=c11", "-fPIC", "-shared")  # gcc; no fast-math, no vectorisation flags


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (BUILD_FLAGS)."""
    if os.environ.get("BKV_ORACLE_LIB"):
        return _LIB  # built by whoever named it
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *BUILD_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        LONG = ctypes.c_long
        L.orc_bf16_from_double.argtypes = [D]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_fps.argtypes = [P, I, I, I, P]
        L.orc_fps.restype = I
        L.orc_fps_objectives.argtypes = [P, I, I, P, I, P]
        L.orc_fps_objectives.restype = None
        L.orc_fps_stored.argtypes = [P, I, I, I, I, P]
        L.orc_fps_stored.restype = I
        L.orc_fps_full.argtypes = [P, I, I, I, I, P]
        L.orc_fps_full.restype = I
        L.orc_fps_full_objectives.argtypes = [P, I, I, I, P, I, P]
        L.orc_fps_full_objectives.restype = None
        L.orc_fps_ingest.argtypes = [P, I, I, I, I, P, P, I]
        L.orc_fps_ingest.restype = I
        L.orc_rope.argtypes = [P, I, LONG, D, P]
        L.orc_rope.restype = None
        L.orc_score_unit.argtypes = [I, I, I, P, I, P, P, I, P, P, I, I, LONG, D, P, P, P, P]
        L.orc_score_unit.restype = I
        L.orc_score_given.argtypes = [I, I, I, P, I, P, P, I, P, P, I, LONG, D, I, P, P, P, P]
        L.orc_score_given.restype = I
        L.orc_decode_attention.argtypes = [I, I, I, P, P, I, P, P, P]
        L.orc_decode_attention.restype = None
        L.orc_capture_step.argtypes = [I, I, I, P, I, P, P]
        L.orc_capture_step.restype = None
        L.orc_score_capture.argtypes = [I, I, I, P, I, P, P, I, I, LONG, D, P, P]
        L.orc_score_capture.restype = I
        L.orc_select.argtypes = [P, I, I, I, P]
        L.orc_select.restype = I
        L.orc_compact.argtypes = [P, LONG, P, I]
        L.orc_compact.restype = None
        L.orc_select_fill.argtypes = [P, P, I, I, I, P]
        L.orc_select_fill.restype = I
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("storage arrays must be float32 or uint16 (bfloat16 bits), got %s" % a.dtype)


def to_double(a: np.ndarray) -> np.ndarray:
    """Exact widening of a storage array to float64."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise TypeError(a.dtype)


# ---------------------------------------------------------------------------
# Element rounding
# ---------------------------------------------------------------------------

def bf16_from_double(v) -> np.ndarray:
    """Single round-to-nearest-even of binary64 values to bfloat16 bits."""
    v = np.asarray(v, dtype=np.float64)
    f = lib().orc_bf16_from_double
    out = np.empty(v.shape, dtype=np.uint16)
    flat_in, flat_out = v.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = f(float(flat_in[i]))
    return out


# ---------------------------------------------------------------------------
# FPS (greedy farthest point sampling on cosine similarity)
# ---------------------------------------------------------------------------

def fps(X: np.ndarray, k: int) -> np.ndarray:
    """FPS picks (pick order) of up to k rows of the float64 matrix X[c, d]."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    c, d = X.shape
    picks = np.empty(max(k, 1), dtype=np.int32)
    n = lib().orc_fps(_ptr(X), c, d, k, _ptr(picks))
    return picks[:n].copy()


def fps_objectives(X: np.ndarray, prefix) -> np.ndarray:
    """Per-row FPS objective given the picked prefix: the mean cosine to all
    rows for an empty prefix, else the maximum cosine to the prefix."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    c, d = X.shape
    pre = np.ascontiguousarray(np.asarray(prefix, dtype=np.int32).reshape(-1))
    out = np.empty(max(c, 1), dtype=np.float64)
    lib().orc_fps_objectives(_ptr(X), c, d, _ptr(pre) if pre.size else None, int(pre.size), _ptr(out))
    return out[:c].copy()


def check_fps_sequence(X: np.ndarray, picks, tol: float, objectives=None):
    """Checks that ``picks`` is a valid FPS run over the rows of X: every pick
    is an unpicked row whose objective is within ``tol`` of the round's
    minimum.  Returns the largest excess over the minimum.  ``objectives``
    (default fps_objectives) maps (X, prefix) to the per-row objective."""
    objectives = objectives or fps_objectives
    picked = np.zeros(X.shape[0], dtype=bool)
    worst = 0.0
    for t, p in enumerate(picks):
        obj = objectives(X, list(picks[:t]))
        assert not picked[p], "row %d picked twice" % p
        best = np.min(obj[~picked])
        excess = obj[p] - best
        assert excess <= tol, "round %d: pick %d objective %r exceeds the minimum %r" % (t, p, obj[p], best)
        worst = max(worst, excess)
        picked[p] = True
    return worst


def fps_stored(buf: np.ndarray, count: int, k: int) -> np.ndarray:
    """FPS picks over the first ``count`` rows of a storage buffer [C, d]."""
    buf = np.ascontiguousarray(buf)
    d = buf.shape[-1]
    picks = np.empty(max(k, 1), dtype=np.int32)
    n = lib().orc_fps_stored(_ptr(buf), dtype_code(buf), count, d, k, _ptr(picks))
    return picks[:n].copy()


def fps_full(X: np.ndarray, k: int) -> np.ndarray:
    """Naive FPS picks (pick order) of up to k rows of a head's whole stored
    query history X [c, d] (storage dtype)."""
    X = np.ascontiguousarray(X)
    c, d = X.shape
    picks = np.empty(max(k, 1), dtype=np.int32)
    n = lib().orc_fps_full(_ptr(X), dtype_code(X), c, d, k, _ptr(picks))
    return picks[:n].copy()


def fps_full_objectives(X: np.ndarray, prefix) -> np.ndarray:
    """fps_objectives for a stored history X [c, d], with the start rule's mean
    similarity taken through the summed normalised row (as fps_full does)."""
    X = np.ascontiguousarray(X)
    c, d = X.shape
    pre = np.ascontiguousarray(np.asarray(prefix, dtype=np.int32).reshape(-1))
    out = np.empty(max(c, 1), dtype=np.float64)
    lib().orc_fps_full_objectives(_ptr(X), dtype_code(X), c, d, _ptr(pre) if pre.size else None, int(pre.size),
                                  _ptr(out))
    return out[:c].copy()


def fps_ingest(buf: np.ndarray, count: int, q_new: np.ndarray, M: int) -> int:
    """Continual FPS of one head, in place on ``buf`` [C, d]; returns the new count."""
    assert buf.flags["C_CONTIGUOUS"] and q_new.flags["C_CONTIGUOUS"]
    assert buf.dtype == q_new.dtype
    C, d = buf.shape
    T = q_new.shape[0]
    cnt = ctypes.c_int(int(count))
    rc = lib().orc_fps_ingest(_ptr(buf), dtype_code(buf), d, C, M, ctypes.byref(cnt), _ptr(q_new), T)
    if rc != 0:
        raise ValueError("oracle fps_ingest rejected count=%d C=%d M=%d" % (count, C, M))
    return cnt.value


def fps_update(q_new: np.ndarray, qbuf: np.ndarray, qcount: np.ndarray, M: int) -> None:
    """Continual FPS of every head: q_new [N,Hq,T,d], qbuf [N,Hq,C,d], qcount [N,Hq] (in place)."""
    N, Hq = qcount.shape
    for n in range(N):
        for g in range(Hq):
            b = np.ascontiguousarray(qbuf[n, g])
            qcount[n, g] = fps_ingest(b, int(qcount[n, g]), np.ascontiguousarray(q_new[n, g]), M)
            qbuf[n, g] = b


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate-half RoPE of one float64 vector (unrounded binary64 result)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib().orc_rope(_ptr(x), x.shape[0], int(pos), float(theta), _ptr(y))
    return y


# ---------------------------------------------------------------------------
# Scoring
# ---------------------------------------------------------------------------

def score_unit(K: np.ndarray, L: int, recent: np.ndarray, recent_pos: np.ndarray,
               qbuf: np.ndarray, qcount: np.ndarray, nb: int, pos_now: int, theta: float):
    """Scores of one (slot, KV head).

    K [>=L, d] storage; recent [G, R, d]; recent_pos [R]; qbuf [G, C, d]; qcount [G].
    Returns (scores float64 [L], obs rows [G*(R+nb), d] storage, valid int32 [rows],
    lse float64 [rows]).
    """
    K = np.ascontiguousarray(K)
    recent = np.ascontiguousarray(recent)
    qbuf = np.ascontiguousarray(qbuf)
    rp = np.ascontiguousarray(recent_pos, dtype=np.int32)
    qc = np.ascontiguousarray(qcount, dtype=np.int32)
    G, R, d = recent.shape
    C = qbuf.shape[1]
    dt = dtype_code(K)
    assert dtype_code(recent) == dt and dtype_code(qbuf) == dt
    rows = G * (R + nb)
    scores = np.zeros(max(L, 1), dtype=np.float64)
    obs = np.zeros((max(rows, 1), d), dtype=K.dtype)
    valid = np.zeros(max(rows, 1), dtype=np.int32)
    lse = np.zeros(max(rows, 1), dtype=np.float64)
    rc = lib().orc_score_unit(dt, d, G, _ptr(K), L, _ptr(recent), _ptr(rp), R, _ptr(qbuf), _ptr(qc),
                              C, nb, int(pos_now), float(theta), _ptr(scores), _ptr(obs), _ptr(valid), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle score rejected a query count")
    return scores[:L].copy(), obs[:rows].copy(), valid[:rows].copy(), lse[:rows].copy()


AGG_MAX = 0
AGG_MEAN = 1


def score_given(K: np.ndarray, L: int, recent: np.ndarray, recent_pos: np.ndarray, brows: np.ndarray,
                bcount: np.ndarray, pos_now: int, theta: float, agg: int = AGG_MAX):
    """Scores of one (slot, KV head) with given beacon rows and a choice of
    aggregation (AGG_MAX or AGG_MEAN over the present rows).

    K [>=L, d] storage; recent [G, R, d]; recent_pos [R]; brows [G, nb, d]
    storage; bcount [G] (rows [0, bcount[g]) of head g are its beacons).
    Returns (scores float64 [L], obs rows [G*(R+nb), d], valid [rows], lse [rows]).
    """
    K = np.ascontiguousarray(K)
    recent = np.ascontiguousarray(recent)
    brows = np.ascontiguousarray(brows)
    rp = np.ascontiguousarray(recent_pos, dtype=np.int32)
    bc = np.ascontiguousarray(bcount, dtype=np.int32)
    G, R, d = recent.shape
    nb = brows.shape[1]
    dt = dtype_code(K)
    assert dtype_code(recent) == dt and dtype_code(brows) == dt
    rows = G * (R + nb)
    scores = np.zeros(max(L, 1), dtype=np.float64)
    obs = np.zeros((max(rows, 1), d), dtype=K.dtype)
    valid = np.zeros(max(rows, 1), dtype=np.int32)
    lse = np.zeros(max(rows, 1), dtype=np.float64)
    rc = lib().orc_score_given(dt, d, G, _ptr(K), L, _ptr(recent), _ptr(rp), R, _ptr(brows), _ptr(bc), nb,
                               int(pos_now), float(theta), int(agg), _ptr(scores), _ptr(obs), _ptr(valid), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle score_given rejected a beacon count")
    return scores[:L].copy(), obs[:rows].copy(), valid[:rows].copy(), lse[:rows].copy()


def decode_attention(K: np.ndarray, V: np.ndarray, L: int, q: np.ndarray):
    """One decode step of one KV head: q [G, d] storage (rotated), K, V
    [>=L, d] storage.  Returns (out float64 [G, d], probs float64 [G, L])."""
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    q = np.ascontiguousarray(q)
    G, d = q.shape
    dt = dtype_code(K)
    assert dtype_code(V) == dt and dtype_code(q) == dt
    out = np.zeros((G, d), dtype=np.float64)
    probs = np.zeros((G, max(L, 1)), dtype=np.float64)
    lib().orc_decode_attention(dt, d, G, _ptr(K), _ptr(V), L, _ptr(q), _ptr(probs), _ptr(out))
    return out, probs[:, :L].copy()


def capture_step(K: np.ndarray, L: int, q: np.ndarray, capture: np.ndarray) -> None:
    """Folds one decode step into a KV head's capture, in place: capture[j] =
    max(capture[j], max_g p_g(j)) for j < L.  q [G, d] storage (rotated), K
    [>=L, d] storage, capture float64 [>=L]."""
    K = np.ascontiguousarray(K)
    q = np.ascontiguousarray(q)
    assert capture.dtype == np.float64 and capture.flags["C_CONTIGUOUS"] and capture.shape[0] >= L
    G, d = q.shape
    dt = dtype_code(K)
    assert dtype_code(q) == dt
    lib().orc_capture_step(dt, d, G, _ptr(K), L, _ptr(q), _ptr(capture))


def score_capture(K: np.ndarray, L: int, qbuf: np.ndarray, qcount: np.ndarray, nb: int, pos_now: int, theta: float,
                  capture: np.ndarray) -> np.ndarray:
    """Eviction scores of one KV head from its beacon rows (FPS of the
    buffers, rotated to pos_now) raised to the captured recent maxima.
    qbuf [G, C, d] storage; qcount [G]; capture float64 [>=L].  Returns
    float64 [L]."""
    K = np.ascontiguousarray(K)
    qbuf = np.ascontiguousarray(qbuf)
    qc = np.ascontiguousarray(qcount, dtype=np.int32)
    cap = np.ascontiguousarray(capture, dtype=np.float64)
    assert cap.shape[0] >= L
    G, C, d = qbuf.shape
    dt = dtype_code(K)
    assert dtype_code(qbuf) == dt
    scores = np.zeros(max(L, 1), dtype=np.float64)
    rc = lib().orc_score_capture(dt, d, G, _ptr(K), L, _ptr(qbuf), _ptr(qc), C, nb, int(pos_now), float(theta),
                                 _ptr(cap), _ptr(scores))
    if rc != 0:
        raise ValueError("oracle score_capture rejected a query count")
    return scores[:L].copy()


def score(K, lens, recent, recent_pos, qbuf, qcount, nb, pos_now, theta, units=None):
    """Scores of many units.  K [N,Hkv,Lmax,d]; lens [N]; recent [N,Hq,R,d];
    recent_pos [N,R]; qbuf [N,Hq,C,d]; qcount [N,Hq]; pos_now [N].

    ``units`` is an iterable of (n, h) pairs (default: all).  Returns a dict
    (n, h) -> (scores, obs, valid, lse).
    """
    N, Hkv = K.shape[0], K.shape[1]
    Hq = recent.shape[1]
    G = Hq // Hkv
    if units is None:
        units = [(n, h) for n in range(N) for h in range(Hkv)]
    out = {}
    for n, h in units:
        g0 = h * G
        out[(n, h)] = score_unit(K[n, h], int(lens[n]), recent[n, g0:g0 + G], recent_pos[n],
                                 qbuf[n, g0:g0 + G], qcount[n, g0:g0 + G], nb, int(pos_now[n]), theta)
    return out


# ---------------------------------------------------------------------------
# Selection and compaction
# ---------------------------------------------------------------------------

def select(scores: np.ndarray, L: int, B: int, W: int) -> np.ndarray:
    """Ascending kept indices (window + top-(B-W), lower index wins ties)."""
    s = np.ascontiguousarray(scores[:L], dtype=np.float64)
    kept = np.empty(max(min(L, B), 1), dtype=np.int32)
    n = lib().orc_select(_ptr(s), L, B, W, _ptr(kept))
    if n < 0:
        raise ValueError("oracle select rejected B=%d W=%d" % (B, W))
    return kept[:n].copy()


def compact(X: np.ndarray, kept: np.ndarray) -> None:
    """In-place gather X[i] <- X_old[kept[i]] of the rows of X [Lmax, d]
    (storage), or of the entries of a 1-D array (positions)."""
    assert X.flags["C_CONTIGUOUS"]
    k = np.ascontiguousarray(kept, dtype=np.int32)
    row_bytes = (X.shape[-1] if X.ndim > 1 else 1) * X.itemsize
    lib().orc_compact(_ptr(X), row_bytes, _ptr(k), int(k.shape[0]))


def select_fill(scores: np.ndarray, pos: np.ndarray, L: int, B: int, W: int) -> np.ndarray:
    """Gather map of the hole-filling layout: the window is the W newest
    positions, the other B-W rows the top scores (older position, then lower
    row, first at ties); evicted rows of [0, B) take the kept rows of [B, L)
    in ascending order.  kept[i] = pre-eviction row that row i holds."""
    s = np.ascontiguousarray(scores[:L], dtype=np.float64)
    p = np.ascontiguousarray(pos[:L], dtype=np.int64)
    assert p.dtype.itemsize == ctypes.sizeof(ctypes.c_long)
    kept = np.empty(max(min(L, B), 1), dtype=np.int32)
    n = lib().orc_select_fill(_ptr(s), _ptr(p), L, B, W, _ptr(kept))
    if n < 0:
        raise ValueError("oracle select_fill rejected B=%d W=%d" % (B, W))
    return kept[:n].copy()


def evict(K, V, lens, scores_by_unit, B, W):
    """Select + compact every unit of K, V [N,Hkv,Lmax,d] in place; returns
    kept dict (n,h) -> indices and the new lengths."""
    N, Hkv = K.shape[0], K.shape[1]
    kept = {}
    new_len = np.array(lens, dtype=np.int32).copy()
    for n in range(N):
        L = int(lens[n])
        for h in range(Hkv):
            k = select(scores_by_unit[(n, h)], L, B, W)
            kept[(n, h)] = k
            kb = np.ascontiguousarray(K[n, h])
            vb = np.ascontiguousarray(V[n, h])
            compact(kb, k)
            compact(vb, k)
            K[n, h] = kb
            V[n, h] = vb
        new_len[n] = min(L, B)
    return kept, new_len
