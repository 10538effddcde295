"""ctypes binding of libbkv.so (argument marshalling only).

Each ``bkv_*`` function mirrors the C entry point of the same name declared
in ``include/bkv.h``: torch tensors become device pointers, the stream
defaults to torch's current stream, and a non-zero status raises
``BkvError``.  No computation happens here, and there is no fallback: if the
library is missing, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbkv.so")

F32 = 0
BF16 = 1

OK = 0
E_NULL, E_SHAPE, E_DTYPE, E_BUDGET, E_CAPACITY, E_WORKSPACE, E_HIP, E_SCRATCH = range(1, 9)
NOALLOC_MAX_UNITS = 131040  # bkv_select_compact_noalloc: (slot, KV head) units its scratch holds
DEV_BAD_LEN = 0x1
DEV_BAD_COUNT = 0x2
DEV_BAD_INDEX = 0x4
AGG_MAX, AGG_MEAN = 0, 1

WS_OBS, WS_VALID, WS_LSE, WS_SELECT, WS_ROPE, WS_BEACONS, WS_BEACON_ROWS = range(7)
WS_HEADER_BYTES = 256

EXPORTS = (
    "bkv_workspace_size",
    "bkv_workspace_layout",
    "bkv_fps_update",
    "bkv_score",
    "bkv_beacon_picks",
    "bkv_score_picked",
    "bkv_score_picked_agg",
    "bkv_beacon_rows",
    "bkv_select",
    "bkv_compact",
    "bkv_select_compact",
    "bkv_select_compact_noalloc",
    "bkv_select_fill",
    "bkv_compact_fill",
    "bkv_select_compact_fill",
    "bkv_decode_workspace_size",
    "bkv_decode_attention",
    "bkv_score_picked_capture",
    "bkv_fps_full_workspace_size",
    "bkv_fps_full",
    "bkv_status_string",
    "bkv_read_device_status",
    "bkv_reset_device_status",
    "bkv_set_debug_copies",
)


class BkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libbkv status %d: %s" % (status, msg))
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libbkv.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libbkv.so is not built (%s); run `python -c \"import __graft_entry__ as g; g.build()\"` "
            "or `python kv_cache_eviction_continual_amd/build.py`" % LIB_PATH
        )
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    L.bkv_workspace_size.argtypes = [SP, I32, I32]
    L.bkv_workspace_size.restype = SZ
    L.bkv_workspace_layout.argtypes = [SP, I32, I32, ctypes.POINTER(SZ)]
    L.bkv_workspace_layout.restype = ctypes.c_int
    L.bkv_fps_update.argtypes = [SP, P, I32, P, P, I32, I32, P, SZ, P]
    L.bkv_fps_update.restype = ctypes.c_int
    L.bkv_score.argtypes = [SP, P, P, P, P, I32, P, P, I32, I32, P, ctypes.c_double, P, P, SZ, P]
    L.bkv_score.restype = ctypes.c_int
    L.bkv_beacon_picks.argtypes = [SP, P, P, I32, I32, I32, P, SZ, P]
    L.bkv_beacon_picks.restype = ctypes.c_int
    L.bkv_score_picked.argtypes = [SP, P, P, P, P, I32, I32, P, ctypes.c_double, P, P, SZ, P]
    L.bkv_score_picked.restype = ctypes.c_int
    L.bkv_select.argtypes = [SP, P, P, I32, I32, P, P, SZ, P]
    L.bkv_select.restype = ctypes.c_int
    L.bkv_compact.argtypes = [SP, P, P, P, I32, P, P, SZ, P]
    L.bkv_compact.restype = ctypes.c_int
    L.bkv_select_compact.argtypes = [SP, P, P, P, P, I32, I32, P, P, SZ, P]
    L.bkv_select_compact.restype = ctypes.c_int
    L.bkv_select_compact_noalloc.argtypes = [SP, P, P, P, P, I32, I32, P, P, P]
    L.bkv_select_compact_noalloc.restype = ctypes.c_int
    L.bkv_select_fill.argtypes = [SP, P, P, P, I32, I32, P, P, SZ, P]
    L.bkv_select_fill.restype = ctypes.c_int
    L.bkv_compact_fill.argtypes = [SP, P, P, P, P, I32, P, P, SZ, P]
    L.bkv_compact_fill.restype = ctypes.c_int
    L.bkv_select_compact_fill.argtypes = [SP, P, P, P, P, P, I32, I32, P, P, SZ, P]
    L.bkv_select_compact_fill.restype = ctypes.c_int
    L.bkv_score_picked_agg.argtypes = [SP, P, P, P, P, I32, I32, P, ctypes.c_double, I32, P, P, SZ, P]
    L.bkv_score_picked_agg.restype = ctypes.c_int
    L.bkv_beacon_rows.argtypes = [SP, P, I32, P, I32, I32, P, SZ, P]
    L.bkv_beacon_rows.restype = ctypes.c_int
    L.bkv_decode_workspace_size.argtypes = [SP]
    L.bkv_decode_workspace_size.restype = SZ
    L.bkv_decode_attention.argtypes = [SP, P, P, P, P, P, P, P, SZ, P]
    L.bkv_decode_attention.restype = ctypes.c_int
    L.bkv_score_picked_capture.argtypes = [SP, P, P, P, I32, P, ctypes.c_double, P, P, SZ, P]
    L.bkv_score_picked_capture.restype = ctypes.c_int
    L.bkv_fps_full_workspace_size.argtypes = [SP, I32]
    L.bkv_fps_full_workspace_size.restype = SZ
    L.bkv_fps_full.argtypes = [SP, P, I32, I32, P, P, SZ, P]
    L.bkv_fps_full.restype = ctypes.c_int
    L.bkv_status_string.argtypes = [ctypes.c_int]
    L.bkv_status_string.restype = ctypes.c_char_p
    L.bkv_set_debug_copies.argtypes = [I32]
    L.bkv_set_debug_copies.restype = I32
    L.bkv_read_device_status.argtypes = [P, ctypes.POINTER(I32), P]
    L.bkv_read_device_status.restype = ctypes.c_int
    L.bkv_reset_device_status.argtypes = [P, P]
    L.bkv_reset_device_status.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != OK:
        raise BkvError(status, load().bkv_status_string(status).decode())


def _storage_dtype(shape: Shape):
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32 if shape.dtype == F32 else None


def _count(*dims) -> int:
    n = 1
    for x in dims:
        n *= max(0, int(x))
    return n


class _Arg:
    """A tensor argument that passed the structural checks of _dev."""

    __slots__ = ("t", "name")

    def __init__(self, t, name):
        self.t, self.name = t, name


def _dev(t, name: str, dtype, numel: int, optional: bool = False):
    """Tensor argument `name` after the checks the C ABI cannot make: a
    dense tensor of the element type the header states, holding at least the
    `numel` elements the call will touch.  None stays None (NULL) when the
    argument is optional; the library then checks whether the call needs it.
    Where it lives is checked by _on_gpu, once every argument has passed
    these checks."""
    if t is None:
        if optional:
            return None
        raise ValueError("%s: a tensor is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor, got %s" % (name, type(t).__name__))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous (dense row-major)" % name)
    if t.numel() < numel:
        raise ValueError("%s: holds %d elements, the call needs %d" % (name, t.numel(), numel))
    return _Arg(t, name)


def _ws(ws, name: str = "ws"):
    """A workspace argument: a dense uint8 tensor (its size and alignment are
    checked by the library, which receives its byte count)."""
    return _dev(ws, name, torch.uint8, 0)


def _on_gpu(*args):
    """Device pointers of checked arguments (None for NULL), each on the
    current GPU."""
    out = []
    for a in args:
        if a is None:
            out.append(None)
            continue
        t = a.t
        if not t.is_cuda:
            raise ValueError("%s: must be on the GPU, got device %s" % (a.name, t.device))
        if t.device.index != torch.cuda.current_device():
            raise ValueError("%s: on %s, but the current device is cuda:%d" % (a.name, t.device,
                                                                              torch.cuda.current_device()))
        out.append(t.data_ptr())
    return out


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return BF16
    if t == torch.float32:
        return F32
    raise TypeError("storage must be bfloat16 or float32, got %s" % t)


def make_shape(n_seq: int, n_kv_heads: int, n_q_heads: int, head_dim: int, max_len: int, dtype) -> Shape:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return Shape(n_seq, n_kv_heads, n_q_heads, head_dim, max_len, code)


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def bkv_workspace_size(shape: Shape, R: int, nb: int) -> int:
    return int(load().bkv_workspace_size(ctypes.byref(shape), R, nb))


def bkv_workspace_layout(shape: Shape, R: int, nb: int):
    offs = (ctypes.c_size_t * 7)()
    _check(load().bkv_workspace_layout(ctypes.byref(shape), R, nb, offs))
    return [int(o) for o in offs]


def _nbytes(ws) -> int:
    return ws.numel()  # uint8: one byte per element


def bkv_fps_update(shape: Shape, q_new, T: int, qbuf, qcount, C: int, M: int, ws, stream=None) -> None:
    N, Hq, d, st = shape.n_seq, shape.n_q_heads, shape.head_dim, _storage_dtype(shape)
    qn, qb, qc, w = _on_gpu(_dev(q_new, "q_new", st, _count(N, Hq, T, d), optional=T <= 0),
                            *_buffers(shape, qbuf, qcount, C), _ws(ws))
    _check(load().bkv_fps_update(ctypes.byref(shape), qn, T, qb, qc, C, M, w, _nbytes(ws), _stream(stream)))


def _score_common(shape: Shape, K, length, recent, recent_pos, R: int, pos_now, scores):
    """The arguments every scoring call shares, checked."""
    N, Hkv, Hq, d, Lmax, st = (shape.n_seq, shape.n_kv_heads, shape.n_q_heads, shape.head_dim, shape.max_len,
                               _storage_dtype(shape))
    return (_dev(K, "K", st, _count(N, Hkv, Lmax, d)), _dev(length, "len", torch.int32, _count(N)),
            _dev(recent, "recent", st, _count(N, Hq, R, d), optional=R <= 0),
            _dev(recent_pos, "recent_pos", torch.int32, _count(N, R), optional=R <= 0),
            _dev(pos_now, "pos_now", torch.int32, _count(N)),
            _dev(scores, "scores", torch.float32, _count(N, Hkv, Lmax)))


def _buffers(shape: Shape, qbuf, qcount, C: int):
    N, Hq, d = shape.n_seq, shape.n_q_heads, shape.head_dim
    return (_dev(qbuf, "qbuf", _storage_dtype(shape), _count(N, Hq, C, d)),
            _dev(qcount, "qcount", torch.int32, _count(N, Hq)))


def bkv_score(shape: Shape, K, length, recent, recent_pos, R: int, qbuf, qcount, C: int, nb: int, pos_now,
              rope_theta: float, scores, ws, stream=None) -> None:
    k, ln, rc, rp, pn, sc, qb, qc, w = _on_gpu(*_score_common(shape, K, length, recent, recent_pos, R, pos_now, scores),
                                               *_buffers(shape, qbuf, qcount, C), _ws(ws))
    _check(load().bkv_score(ctypes.byref(shape), k, ln, rc, rp, R, qb, qc, C, nb, pn, float(rope_theta), sc, w,
                            _nbytes(ws), _stream(stream)))


def bkv_beacon_picks(shape: Shape, qbuf, qcount, C: int, R: int, nb: int, ws, stream=None) -> None:
    qb, qc, w = _on_gpu(*_buffers(shape, qbuf, qcount, C), _ws(ws))
    _check(load().bkv_beacon_picks(ctypes.byref(shape), qb, qc, C, R, nb, w, _nbytes(ws), _stream(stream)))


def bkv_score_picked(shape: Shape, K, length, recent, recent_pos, R: int, nb: int, pos_now, rope_theta: float,
                     scores, ws, stream=None) -> None:
    k, ln, rc, rp, pn, sc, w = _on_gpu(*_score_common(shape, K, length, recent, recent_pos, R, pos_now, scores),
                                       _ws(ws))
    _check(load().bkv_score_picked(ctypes.byref(shape), k, ln, rc, rp, R, nb, pn, float(rope_theta), sc, w,
                                   _nbytes(ws), _stream(stream)))


def bkv_score_picked_agg(shape: Shape, K, length, recent, recent_pos, R: int, nb: int, pos_now, rope_theta: float,
                         aggregation: int, scores, ws, stream=None) -> None:
    k, ln, rc, rp, pn, sc, w = _on_gpu(*_score_common(shape, K, length, recent, recent_pos, R, pos_now, scores),
                                       _ws(ws))
    _check(load().bkv_score_picked_agg(ctypes.byref(shape), k, ln, rc, rp, R, nb, pn, float(rope_theta),
                                       int(aggregation), sc, w, _nbytes(ws), _stream(stream)))


def bkv_beacon_rows(shape: Shape, src, S: int, idx, R: int, nb: int, ws, stream=None) -> None:
    N, Hq, d = shape.n_seq, shape.n_q_heads, shape.head_dim
    sr, ix, w = _on_gpu(_dev(src, "src", _storage_dtype(shape), _count(N, Hq, S, d), optional=S <= 0 or nb <= 0),
                        _dev(idx, "idx", torch.int32, _count(N, Hq, nb), optional=nb <= 0), _ws(ws))
    _check(load().bkv_beacon_rows(ctypes.byref(shape), sr, S, ix, R, nb, w, _nbytes(ws), _stream(stream)))


def _select_common(shape: Shape, scores, length, budget: int, kept):
    N, Hkv, Lmax = shape.n_seq, shape.n_kv_heads, shape.max_len
    return (_dev(scores, "scores", torch.float32, _count(N, Hkv, Lmax)), _dev(length, "len", torch.int32, _count(N)),
            _dev(kept, "kept", torch.int32, _count(N, Hkv, budget)))


def _kv(shape: Shape, K, V):
    n = _count(shape.n_seq, shape.n_kv_heads, shape.max_len, shape.head_dim)
    st = _storage_dtype(shape)
    return _dev(K, "K", st, n), _dev(V, "V", st, n)


def _len_kept(shape: Shape, length, budget: int, kept):
    return (_dev(length, "len", torch.int32, _count(shape.n_seq)),
            _dev(kept, "kept", torch.int32, _count(shape.n_seq, shape.n_kv_heads, budget)))


def _positions(shape: Shape, pos):
    return _dev(pos, "pos", torch.int32, _count(shape.n_seq, shape.n_kv_heads, shape.max_len))


def bkv_select(shape: Shape, scores, length, budget: int, window: int, kept, ws, stream=None) -> None:
    sc, ln, kp, w = _on_gpu(*_select_common(shape, scores, length, budget, kept), _ws(ws))
    _check(load().bkv_select(ctypes.byref(shape), sc, ln, budget, window, kp, w, _nbytes(ws), _stream(stream)))


def bkv_compact(shape: Shape, K, V, length, budget: int, kept, ws, stream=None) -> None:
    k, v, ln, kp, w = _on_gpu(*_kv(shape, K, V), *_len_kept(shape, length, budget, kept), _ws(ws))
    _check(load().bkv_compact(ctypes.byref(shape), k, v, ln, budget, kp, w, _nbytes(ws), _stream(stream)))


def bkv_select_compact(shape: Shape, scores, K, V, length, budget: int, window: int, kept, ws, stream=None) -> None:
    sc, ln, kp, k, v, w = _on_gpu(*_select_common(shape, scores, length, budget, kept), *_kv(shape, K, V), _ws(ws))
    _check(load().bkv_select_compact(ctypes.byref(shape), sc, k, v, ln, budget, window, kp, w, _nbytes(ws),
                                     _stream(stream)))


def bkv_select_compact_noalloc(shape: Shape, scores, K, V, length, budget: int, window: int, kept,
                               dev_status=None, stream=None) -> None:
    sc, ln, kp, k, v, so = _on_gpu(*_select_common(shape, scores, length, budget, kept), *_kv(shape, K, V),
                                   _dev(dev_status, "dev_status", torch.int32, 1, optional=True))
    _check(load().bkv_select_compact_noalloc(ctypes.byref(shape), sc, k, v, ln, budget, window, kp, so,
                                             _stream(stream)))


def bkv_select_fill(shape: Shape, scores, pos, length, budget: int, window: int, kept, ws, stream=None) -> None:
    sc, ln, kp, ps, w = _on_gpu(*_select_common(shape, scores, length, budget, kept), _positions(shape, pos),
                                _ws(ws))
    _check(load().bkv_select_fill(ctypes.byref(shape), sc, ps, ln, budget, window, kp, w, _nbytes(ws),
                                  _stream(stream)))


def bkv_compact_fill(shape: Shape, K, V, pos, length, budget: int, kept, ws, stream=None) -> None:
    k, v, ps, ln, kp, w = _on_gpu(*_kv(shape, K, V), _positions(shape, pos), *_len_kept(shape, length, budget, kept),
                                  _ws(ws))
    _check(load().bkv_compact_fill(ctypes.byref(shape), k, v, ps, ln, budget, kp, w, _nbytes(ws), _stream(stream)))


def bkv_select_compact_fill(shape: Shape, scores, K, V, pos, length, budget: int, window: int, kept, ws,
                            stream=None) -> None:
    sc, ln, kp, k, v, ps, w = _on_gpu(*_select_common(shape, scores, length, budget, kept), *_kv(shape, K, V),
                                      _positions(shape, pos), _ws(ws))
    _check(load().bkv_select_compact_fill(ctypes.byref(shape), sc, k, v, ps, ln, budget, window, kp, w, _nbytes(ws),
                                          _stream(stream)))


def bkv_decode_workspace_size(shape: Shape) -> int:
    return int(load().bkv_decode_workspace_size(ctypes.byref(shape)))


def bkv_decode_attention(shape: Shape, q, K, V, length, out, capture, ws, stream=None) -> None:
    N, Hkv, Hq, d, Lmax = shape.n_seq, shape.n_kv_heads, shape.n_q_heads, shape.head_dim, shape.max_len
    qp, k, v, ln, op, cp, w = _on_gpu(_dev(q, "q", _storage_dtype(shape), _count(N, Hq, d)), *_kv(shape, K, V),
                                      _dev(length, "len", torch.int32, _count(N)),
                                      _dev(out, "out", torch.float32, _count(N, Hq, d)),
                                      _dev(capture, "capture", torch.float32, _count(N, Hkv, Lmax), optional=True),
                                      _ws(ws))
    _check(load().bkv_decode_attention(ctypes.byref(shape), qp, k, v, ln, op, cp, w, _nbytes(ws), _stream(stream)))


def bkv_score_picked_capture(shape: Shape, K, length, capture, nb: int, pos_now, rope_theta: float, scores, ws,
                             stream=None) -> None:
    N, Hkv, Lmax = shape.n_seq, shape.n_kv_heads, shape.max_len
    k, ln, _, _, pn, sc, cp, w = _on_gpu(*_score_common(shape, K, length, None, None, 0, pos_now, scores),
                                         _dev(capture, "capture", torch.float32, _count(N, Hkv, Lmax)), _ws(ws))
    _check(load().bkv_score_picked_capture(ctypes.byref(shape), k, ln, cp, nb, pn, float(rope_theta), sc, w,
                                           _nbytes(ws), _stream(stream)))


def bkv_fps_full_workspace_size(shape: Shape, n: int) -> int:
    return int(load().bkv_fps_full_workspace_size(ctypes.byref(shape), n))


def bkv_fps_full(shape: Shape, hist, n: int, k: int, picks, ws, stream=None) -> None:
    N, Hq, d = shape.n_seq, shape.n_q_heads, shape.head_dim
    hp, pk, w = _on_gpu(_dev(hist, "hist", _storage_dtype(shape), _count(N, Hq, n, d), optional=n <= 0),
                        _dev(picks, "picks", torch.int32, _count(N, Hq, k), optional=k <= 0), _ws(ws))
    _check(load().bkv_fps_full(ctypes.byref(shape), hp, n, k, pk, w, _nbytes(ws), _stream(stream)))


def bkv_set_debug_copies(on: bool) -> bool:
    """Turns the scoring calls' copy of the rotated observation rows (workspace
    region obs) on or off, process-wide; returns the previous setting."""
    return bool(load().bkv_set_debug_copies(1 if on else 0))


def bkv_status_string(status: int) -> str:
    return load().bkv_status_string(status).decode()


def bkv_read_device_status(ws, stream=None) -> int:
    out = ctypes.c_int32(0)
    (w,) = _on_gpu(_ws(ws))
    _check(load().bkv_read_device_status(w, ctypes.byref(out), _stream(stream)))
    return int(out.value)


def bkv_reset_device_status(ws, stream=None) -> None:
    (w,) = _on_gpu(_ws(ws))
    _check(load().bkv_reset_device_status(w, _stream(stream)))


# ---------------------------------------------------------------------------
# Workspace helpers (allocation through torch; views of documented regions)
# ---------------------------------------------------------------------------

def alloc_workspace(shape: Shape, R: int, nb: int, device="cuda") -> torch.Tensor:
    """A zeroed, 256-byte aligned workspace (torch allocations are aligned)."""
    n = bkv_workspace_size(shape, R, nb)
    if n == 0:
        raise BkvError(E_SHAPE, "workspace size is 0 for this shape / R / nb")
    ws = torch.zeros(n, dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def ws_rows_moved(ws) -> int:
    return int(ws[8:16].view(torch.int64).item())


def ws_views(shape: Shape, R: int, nb: int, ws):
    """Typed views of the workspace regions: obs rows, valid flags, lse,
    select table, beacon picks."""
    offs = bkv_workspace_layout(shape, R, nb)
    G = shape.n_q_heads // shape.n_kv_heads
    rows = G * (R + nb)
    RP = (rows + 31) // 32 * 32
    units = shape.n_seq * shape.n_kv_heads
    d = shape.head_dim
    st = torch.bfloat16 if shape.dtype == BF16 else torch.float32
    es = 2 if shape.dtype == BF16 else 4
    obs = ws[offs[WS_OBS]:offs[WS_OBS] + units * RP * d * es].view(st).view(shape.n_seq, shape.n_kv_heads, RP, d)
    valid = ws[offs[WS_VALID]:offs[WS_VALID] + units * RP * 4].view(torch.int32).view(shape.n_seq, shape.n_kv_heads, RP)
    lse = ws[offs[WS_LSE]:offs[WS_LSE] + units * RP * 4].view(torch.float32).view(shape.n_seq, shape.n_kv_heads, RP)
    sel = ws[offs[WS_SELECT]:offs[WS_SELECT] + units * 8].view(torch.int32).view(shape.n_seq, shape.n_kv_heads, 2)
    nbk = shape.n_seq * shape.n_q_heads * (nb + 1)
    beacons = ws[offs[WS_BEACONS]:offs[WS_BEACONS] + nbk * 4].view(torch.int32).view(shape.n_seq, shape.n_q_heads,
                                                                                       nb + 1)
    st_bytes = es * d
    nbr = shape.n_seq * shape.n_q_heads * nb
    brows = ws[offs[WS_BEACON_ROWS]:offs[WS_BEACON_ROWS] + nbr * st_bytes].view(st).view(shape.n_seq, shape.n_q_heads,
                                                                                      nb, d)
    return {"obs": obs, "valid": valid, "lse": lse, "select": sel, "beacons": beacons, "beacon_rows": brows,
            "rows": rows, "RP": RP}
