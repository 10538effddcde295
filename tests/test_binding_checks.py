"""The Python binding refuses, before any call into the library, tensors that
the C ABI cannot vet: a wrong element type, a non-contiguous view, too few
elements for the sizes the header states, or memory that is not on the GPU.
Each case would otherwise hand the kernels a pointer they read or write out
of bounds.  Host tensors stand in for device ones: every check but the last
fires before the device is looked at, and the last one is the device check
itself."""
import pytest
import torch

from kv_cache_eviction_continual_amd import bkv

N, HKV, HQ, D, LMAX, B, W, R, NB, C, M = 2, 2, 4, 64, 96, 64, 8, 3, 4, 16, 4


def shape(dtype=torch.bfloat16):
    return bkv.make_shape(N, HKV, HQ, D, LMAX, dtype)


def good():
    """Host tensors with the right types and sizes for `shape()`."""
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    return {
        "K": torch.zeros(N, HKV, LMAX, D, dtype=bf),
        "V": torch.zeros(N, HKV, LMAX, D, dtype=bf),
        "len": torch.zeros(N, dtype=i32),
        "recent": torch.zeros(N, HQ, R, D, dtype=bf),
        "recent_pos": torch.zeros(N, R, dtype=i32),
        "pos_now": torch.zeros(N, dtype=i32),
        "scores": torch.zeros(N, HKV, LMAX, dtype=f32),
        "qbuf": torch.zeros(N, HQ, C, D, dtype=bf),
        "qcount": torch.zeros(N, HQ, dtype=i32),
        "q_new": torch.zeros(N, HQ, 5, D, dtype=bf),
        "kept": torch.zeros(N, HKV, B, dtype=i32),
        "pos": torch.zeros(N, HKV, LMAX, dtype=i32),
        "ws": torch.zeros(1 << 16, dtype=torch.uint8),
    }


CALLS = {
    "fps_update": lambda t: bkv.bkv_fps_update(shape(), t["q_new"], 5, t["qbuf"], t["qcount"], C, M, t["ws"]),
    "score": lambda t: bkv.bkv_score(shape(), t["K"], t["len"], t["recent"], t["recent_pos"], R, t["qbuf"],
                                     t["qcount"], C, NB, t["pos_now"], 1e4, t["scores"], t["ws"]),
    "score_picked": lambda t: bkv.bkv_score_picked(shape(), t["K"], t["len"], t["recent"], t["recent_pos"], R, NB,
                                                   t["pos_now"], 1e4, t["scores"], t["ws"]),
    "select": lambda t: bkv.bkv_select(shape(), t["scores"], t["len"], B, W, t["kept"], t["ws"]),
    "compact": lambda t: bkv.bkv_compact(shape(), t["K"], t["V"], t["len"], B, t["kept"], t["ws"]),
    "select_compact": lambda t: bkv.bkv_select_compact(shape(), t["scores"], t["K"], t["V"], t["len"], B, W,
                                                       t["kept"], t["ws"]),
    "select_compact_fill": lambda t: bkv.bkv_select_compact_fill(shape(), t["scores"], t["K"], t["V"], t["pos"],
                                                                 t["len"], B, W, t["kept"], t["ws"]),
}

# (call, argument) pairs whose checks are exercised below
ARGS = [(c, a) for c, args in {
    "fps_update": ("q_new", "qbuf", "qcount", "ws"),
    "score": ("K", "len", "recent", "recent_pos", "pos_now", "scores", "qbuf", "qcount", "ws"),
    "score_picked": ("K", "recent", "scores"),
    "select": ("scores", "len", "kept", "ws"),
    "compact": ("K", "V", "len", "kept"),
    "select_compact": ("scores", "K", "V", "kept"),
    "select_compact_fill": ("pos", "kept", "K"),
}.items() for a in args]


def wrong_dtype(t):
    return t.to(torch.int64) if t.dtype != torch.int64 else t.to(torch.int32)


@pytest.mark.parametrize("call,arg", ARGS)
def test_wrong_element_type_refused(call, arg):
    t = good()
    t[arg] = wrong_dtype(t[arg])
    with pytest.raises(TypeError, match=arg if arg != "len" else "len"):
        CALLS[call](t)


@pytest.mark.parametrize("call,arg", [a for a in ARGS if a[1] != "ws"])
def test_non_contiguous_view_refused(call, arg):
    t = good()
    x = t[arg]
    # same element type and count, strided: a transposed copy viewed back
    view = torch.cat([x.flatten(), x.flatten()])[::2] if x.dim() == 1 else x.transpose(0, -1).contiguous().transpose(0, -1)
    assert not view.is_contiguous() and view.numel() == x.numel() and view.dtype == x.dtype
    t[arg] = view
    with pytest.raises(ValueError, match="contiguous"):
        CALLS[call](t)


@pytest.mark.parametrize("call,arg", [a for a in ARGS if a[1] != "ws"])
def test_too_few_elements_refused(call, arg):
    t = good()
    t[arg] = t[arg].flatten()[:-1].clone()
    with pytest.raises(ValueError, match="elements"):
        CALLS[call](t)


@pytest.mark.parametrize("call", sorted(CALLS))
def test_host_memory_refused(call):
    """All types and sizes right: the first tensor checked is refused because
    it is not on the GPU (the library would be handed a host pointer)."""
    with pytest.raises(ValueError, match="GPU"):
        CALLS[call](good())


def test_bf16_storage_under_an_f32_shape_refused():
    t = good()
    with pytest.raises(TypeError, match="K"):
        bkv.bkv_compact(shape(torch.float32), t["K"], t["V"], t["len"], B, t["kept"], t["ws"])


def test_optional_arguments_may_be_absent():
    """recent / recent_pos only when R > 0, q_new only when T > 0: absent ones
    pass the binding (the first present tensor then decides, here the host
    check)."""
    t = good()
    with pytest.raises(ValueError, match="GPU"):
        bkv.bkv_score_picked(shape(), t["K"], t["len"], None, None, 0, NB, t["pos_now"], 1e4, t["scores"], t["ws"])
    with pytest.raises(ValueError, match="recent"):
        bkv.bkv_score_picked(shape(), t["K"], t["len"], None, None, R, NB, t["pos_now"], 1e4, t["scores"], t["ws"])
    with pytest.raises(ValueError, match="qbuf"):
        bkv.bkv_fps_update(shape(), None, 0, t["qbuf"], t["qcount"], C, M, t["ws"])
