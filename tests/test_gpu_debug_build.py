"""The debug build (libsegattn_debug.so: host.cpp with SA_DEBUG_CHECKS) on the GPU.

Release builds trust the device index lists they are given (frame lists and
block lists). The debug build copies each list to the host before the launch
that reads it and refuses entries outside their range (SA_E_RANGE) or a block
list row that repeats a block (SA_E_ARG). It also fills every attention
output row with NaN before the launch, so a row the kernels skip would show.

Every refused case here keeps the kernels' reads inside allocated memory even
if the check were missing: the layer is described to the library with a
smaller frame capacity than its planes hold, and a block index one past the
candidates maps to a frame-list entry that exists (the own segment's frames
follow the history). Valid calls must give the release build's result bit
for bit (the same kernels run).
"""

import ctypes

import numpy as np
import pytest
import torch

import diffusion_transformer_attention_segment_amd as sa
from diffusion_transformer_attention_segment_amd import binding as B
from diffusion_transformer_attention_segment_amd import build
import seeded_inputs as si
from helpers import Session

pytestmark = pytest.mark.gpu

SA_E_ARG, SA_E_RANGE = 1, 5


@pytest.fixture(scope="module")
def dbg():
    return B.load(build.DEBUG_LIB)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shrunk(layer, capacity):
    """A copy of the layer's C description with a smaller frame capacity."""
    L = B.sa_kv_layer.from_buffer_copy(layer.c())
    L.frame_capacity = capacity
    return L


def _attend(lib, s, it):
    g = s.geom.c()
    arr = (B.sa_attn_item * 1)(it)
    return lib.sa_segment_attention(ctypes.byref(g), arr, 1, None, 0, _stream())


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_debug_build_matches_release_bitwise(dbg, kv):
    wl = si.Workload(f"dbg_{kv}", heads=2, lat_t=3, lat_h=8, lat_w=16, n_text=40,
                     prior_segments=(2,), kv_dtype=kv, scale_factors=(kv == "fp8"))
    print(f"debug build vs release, {kv}", flush=True)
    s = Session(wl, seed=141, layer=0, session=0)
    assert _attend(sa.lib(), s, s.item().c()) == 0     # both without a workspace: unsplit
    torch.cuda.synchronize()
    want, want_lse = s.out.clone(), s.lse.clone()
    s.out.zero_()
    s.lse.zero_()
    assert _attend(dbg, s, s.item().c()) == 0, dbg.sa_last_error()
    torch.cuda.synchronize()
    assert torch.equal(s.out.view(torch.int16), want.view(torch.int16))
    assert torch.equal(s.lse.view(torch.int32), want_lse.view(torch.int32))
    assert bool(torch.isfinite(s.out.float()).all())


def test_debug_build_refuses_out_of_range_frames(dbg):
    wl = si.Workload("dbg_frames", heads=2, lat_t=3, lat_h=8, lat_w=16, n_text=40,
                     prior_segments=(2,))
    print("debug build: frame list entry past the described capacity", flush=True)
    s = Session(wl, seed=142, layer=0, session=0)
    cap = wl.frame_capacity(0)
    assert max(s.frames) == cap - 1
    L = _shrunk(s.kv, cap - 1)
    it = s.item().c()
    it.kv = ctypes.pointer(L)
    assert _attend(dbg, s, it) == SA_E_RANGE
    msg = dbg.sa_last_error()
    assert b"debug check" in msg and b"frames" in msg, msg
    # the same call is accepted with the true capacity
    it.kv = ctypes.pointer(s.kv.c())
    assert _attend(dbg, s, it) == 0, dbg.sa_last_error()

    # history_gather and sparse_select read the same kind of list
    g = s.geom.c()
    dst = sa.KVLayer.allocate(s.geom, sa.KV_BF16, cap, 48)
    n = len(s.frames)
    assert dbg.sa_history_gather(ctypes.byref(g), ctypes.byref(L), B._ptr(s.d_frames), n,
                                 ctypes.byref(dst.c()), _stream()) == SA_E_RANGE
    assert dbg.sa_history_gather(ctypes.byref(g), ctypes.byref(s.kv.c()), B._ptr(s.d_frames), n,
                                 ctypes.byref(dst.c()), _stream()) == 0
    sel = s.item().c()
    sel.kv = ctypes.pointer(_shrunk(s.kv, 5))
    sel.n_hist_frames, sel.keep_blocks = 6, 3          # history frames 0..5: entry 5 is refused
    lists = torch.empty((2, 2, 3), dtype=torch.int32, device="cuda")
    ws = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    assert dbg.sa_sparse_select(ctypes.byref(g), ctypes.byref(sel), B._ptr(ws), ws.numel(),
                                B._ptr(lists), _stream()) == SA_E_RANGE
    torch.cuda.synchronize()


def test_debug_build_refuses_bad_block_lists(dbg):
    wl = si.Workload("dbg_lists", heads=2, lat_t=3, lat_h=8, lat_w=16, n_text=40,
                     prior_segments=(2,))
    print("debug build: block list out of range, then repeated", flush=True)
    s = Session(wl, seed=143, layer=0, session=0)
    n_hist = 6                       # 6 history frames x 2 blocks = 12 candidates
    assert len(s.frames) > n_hist
    nq = -(-wl.Lq // sa.SPARSE_QUERY_BLOCK)
    good = np.tile(np.array([0, 3, 7, 11], dtype=np.int32), (wl.heads, nq, 1))
    s.set_sparse(good, n_hist)
    assert _attend(dbg, s, s.item().c()) == 0, dbg.sa_last_error()
    bad = good.copy()
    bad[1, nq - 1, 3] = 12           # one past the candidates
    s.set_sparse(bad, n_hist)
    assert _attend(dbg, s, s.item().c()) == SA_E_RANGE
    assert b"block_list" in dbg.sa_last_error()
    rep = good.copy()
    rep[0, 0, 2] = 0                 # a block listed twice (row [0, 3, 0, 11])
    s.set_sparse(rep, n_hist)
    assert _attend(dbg, s, s.item().c()) == SA_E_ARG
    assert b"repeats" in dbg.sa_last_error()
    torch.cuda.synchronize()
