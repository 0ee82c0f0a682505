"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, validates arguments before any HIP call, and its host-only
history selection agrees bit-exactly with the oracle.

No call here reaches a kernel launch: every case either runs host-only code
(history_select, cache_bytes) or fails validation first.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import diffusion_transformer_attention_segment_amd as sa
from diffusion_transformer_attention_segment_amd import binding as B
from oracle import cache as ocache
from oracle import select as osel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "segattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIB_PATH):
        from diffusion_transformer_attention_segment_amd import build
        build.build()
    return sa.lib()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.SIGNATURES) == declared


def test_debug_library_exports_every_declared_symbol(lib):
    """The debug build (device index lists checked on the host) has the same ABI."""
    from diffusion_transformer_attention_segment_amd import build
    dbg = B.load(build.DEBUG_LIB)
    for name in _declared_functions():
        assert hasattr(dbg, name), name
    assert dbg.sa_abi_version() == sa.abi_version()


def test_abi_version(lib):
    assert sa.abi_version() == 11


def test_binding_constants_match_the_header():
    """The Python binding's limits and sizes are the header's #defines."""
    text = open(HEADER).read()
    defs = {m.group(1): m.group(2) for m in re.finditer(r"#define (SA_[A-Z0-9_]+) +([^/\n]+)", text)}

    def value(name):
        return int(eval(defs[name].strip().replace("u", "")))   # integers and shifts only

    assert value("SA_ABI_VERSION") == sa.abi_version()
    assert value("SA_HEAD_DIM") == sa.HEAD_DIM
    assert value("SA_MAX_ITEMS") == sa.MAX_ITEMS
    assert value("SA_MAX_FRAMES_KV") == sa.MAX_FRAMES_KV
    assert value("SA_MAX_CAMERA_CHUNK") == sa.MAX_CAMERA_CHUNK
    assert value("SA_SPARSE_KEY_BLOCK") == sa.SPARSE_KEY_BLOCK
    assert value("SA_SPARSE_QUERY_BLOCK") == sa.SPARSE_QUERY_BLOCK
    assert value("SA_SPARSE_SCRATCH_BYTES") == sa.SPARSE_SCRATCH_BYTES


def test_status_strings(lib):
    assert lib.sa_status_string(0) == b"SA_OK"
    assert lib.sa_status_string(7) == b"SA_E_HIP"


@pytest.mark.parametrize("policy", ["all", "recent", "power", "anchor"])
def test_history_select_matches_oracle(lib, policy):
    for T in range(0, 400, 7):
        for budget in (1, 2, 3, 7, 18, 40):
            if policy == "all":
                got = sa.history_select(sa.SEL_ALL, T)
                want = osel.select_all(T)
            elif policy == "recent":
                got = sa.history_select(sa.SEL_RECENT, T, budget)
                want = osel.select_recent(T, budget)
            elif policy == "power":
                got = sa.history_select(sa.SEL_POWER, T, budget, 2.0)
                want = osel.select_power(T, budget, 2.0)
            else:
                got = sa.history_select(sa.SEL_ANCHOR_RECENT, T, 0, 2.0, frames_per_segment=budget,
                                        recent_segments=3)
                want = osel.select_anchor_recent(T, budget, 3)
            assert got == want.tolist(), (policy, T, budget)


def test_sparse_keep_matches_oracle(lib):
    """The library's keep count for block-sparse history equals the oracle's
    rule (ceil of the percentage, at least one block, at most all of them),
    bit for bit over a sweep; a percentage outside [1, 100] is refused."""
    from oracle import sparse as osp
    for n in list(range(0, 300)) + [1679, 1680, 3360, 8191, 8192]:
        for pct in (1, 10, 25, 33, 50, 99, 100):
            want = osp.keep_count(n, pct) if n > 0 else 0
            assert lib.sa_sparse_keep(n, pct) == want, (n, pct)
            assert sa.sparse_keep(n, pct) == want
    assert sa.sparse_keep(120 * 14, 25) == 420
    for pct in (0, -5, 101):
        assert lib.sa_sparse_keep(10, pct) == -1
        assert b"percent" in lib.sa_last_error()
        with pytest.raises(B.SegAttnError):
            sa.sparse_keep(10, pct)


def test_history_select_power_printed_example(lib):
    got = sa.history_select(sa.SEL_POWER, 360, 18, 2.0)
    assert got == [0, 40, 78, 113, 146, 177, 205, 231, 254, 275, 294, 310, 324, 336, 345, 352,
                   357, 359]


def test_history_select_power_other_gamma(lib):
    for T in (50, 100, 361):
        for g in (1.0, 1.5, 3.0):
            assert sa.history_select(sa.SEL_POWER, T, 10, g) == osel.select_power(T, 10, g).tolist()


def test_history_select_errors(lib):
    with pytest.raises(sa.SegAttnError) as e:
        sa.history_select(sa.SEL_ALL, 10, cap=5)
    assert e.value.status == 6
    with pytest.raises(sa.SegAttnError) as e:
        sa.history_select(99, 10)
    assert e.value.status == 1
    with pytest.raises(sa.SegAttnError):
        sa.history_select(sa.SEL_ALL, -1)


def test_cache_bytes_matches_oracle(lib):
    g = sa.Geom()
    for dt, name in ((sa.KV_BF16, "bf16"), (sa.KV_FP8, "fp8"), (sa.KV_INT8, "int8")):
        for fc, tc in ((60, 256), (390, 256), (0, 16), (1, 0)):
            assert sa.cache_bytes(g, dt, fc, tc) == ocache.plane_bytes(name, 16, 128, 880, fc, tc)
    # frames of 24 tokens: the one-byte caches count 32 slots per plane
    g24 = sa.Geom(heads=2, lat_h=4, lat_w=6)
    for dt, name in ((sa.KV_BF16, "bf16"), (sa.KV_FP8, "fp8"), (sa.KV_INT8, "int8")):
        assert sa.cache_bytes(g24, dt, 3, 16) == ocache.plane_bytes(name, 2, 128, 24, 3, 16)
    # the page's figures: 8,192 bytes per token per layer in bf16, 4,224 in int8
    assert sa.cache_bytes(g, sa.KV_BF16, 1, 0) == 880 * 8192
    assert sa.cache_bytes(g, sa.KV_INT8, 1, 0) == 880 * 4224


# --------------------------------------------------------------- validation
FAKE = 0x100000     # never dereferenced: validation must fail before any launch


def _layer(dtype=0, fc=4, tc=16, k=FAKE, v=FAKE, kt=FAKE, vt=FAKE, ks=FAKE, vs=FAKE):
    L = B.sa_kv_layer()
    L.dtype, L.frame_capacity, L.text_capacity = dtype, fc, tc
    L.k, L.v, L.k_text, L.v_text = k, v, kt, vt
    L.k_scale, L.v_scale, L.k_text_scale, L.v_text_scale = ks, vs, ks, vs
    return L


def _geom(**kw):
    g = sa.Geom(heads=2, lat_h=4, lat_w=6)
    for k, v in kw.items():
        setattr(g, k, v)
    return g.c()


def _append(g, L, k=FAKE, v=FAKE, f0=0, n=1):
    return sa.lib().sa_kv_append(ctypes.byref(g), ctypes.byref(L), ctypes.c_void_p(k),
                                 ctypes.c_void_p(v), f0, n, None)


def test_validation_errors(lib):
    assert _append(_geom(head_dim=64), _layer()) == 2
    assert _append(_geom(rope_split=(16, 56, 54)), _layer()) == 2
    assert _append(_geom(rope_split=(15, 57, 56)), _layer()) == 2
    assert _append(_geom(lat_w=5), _layer()) == 2                 # P = 20 not a multiple of 8
    assert _append(_geom(rope_theta=1.0), _layer()) == 2
    assert _append(_geom(), _layer(dtype=5)) == 4
    assert _append(_geom(), _layer(k=0)) == 1
    assert _append(_geom(), _layer(k=FAKE + 4)) == 3
    assert _append(_geom(), _layer(tc=8)) == 2                    # text capacity % 16
    # fp8 and int8 layers of 24-token frames pass the layer checks (planes of 32 slots)
    assert _append(_geom(), _layer(dtype=1), n=-1) == 1
    assert b"n_frames" in lib.sa_last_error()
    assert _append(_geom(), _layer(dtype=2), n=-1) == 1
    assert _append(_geom(), _layer(), f0=3, n=2) == 5             # frames 3..4 > capacity 4
    assert _append(_geom(), _layer(), f0=-1) == 5
    assert _append(_geom(), _layer(), k=FAKE + 2) == 3
    assert _append(_geom(), _layer(), n=-1) == 1
    assert b"n_frames" in lib.sa_last_error()
    # the message is cleared by the next successful call
    assert _append(_geom(), _layer(), n=0) == 0
    assert lib.sa_last_error() == b""
    g = _geom()
    assert lib.sa_text_append(ctypes.byref(g), ctypes.byref(_layer()), ctypes.c_void_p(FAKE),
                              ctypes.c_void_p(FAKE), 17, None) == 6
    assert lib.sa_kv_append(None, ctypes.byref(_layer()), None, None, 0, 1, None) == 1


def _item(L, rows=True, n_frames_kv=2, n_text_kv=3, frames=FAKE):
    it = B.sa_attn_item()
    it.q, it.out = FAKE, FAKE
    it.frame0_q, it.n_frames_q, it.n_text_q = 0, 1 if rows else 0, 0
    it.kv = ctypes.pointer(L)
    it.frames = frames
    it.n_frames_kv, it.n_text_kv = n_frames_kv, n_text_kv
    return it


def _attn(items, n=None):
    g = _geom()
    arr = (B.sa_attn_item * max(len(items), 1))(*items)
    return sa.lib().sa_segment_attention(ctypes.byref(g), arr, len(items) if n is None else n,
                                         None, 0, None)


def test_attention_validation(lib):
    L = _layer()
    g = _geom()
    arr = (B.sa_attn_item * 1)(_item(L))
    cnt = lib.sa_segment_attention_counted
    assert cnt(ctypes.byref(g), arr, 1, None, 0, None, None) == 1              # no counters
    assert cnt(ctypes.byref(g), arr, 1, None, 0, ctypes.c_void_p(FAKE + 2), None) == 3
    assert cnt(ctypes.byref(g), arr, 0, None, 0, ctypes.c_void_p(FAKE), None) == 1
    assert _attn([_item(L)], n=0) == 1
    assert _attn([_item(L)] * 9) == 1
    assert _attn([_item(L, n_frames_kv=0, n_text_kv=0)]) == 1     # empty key set
    assert _attn([_item(L, n_text_kv=17)]) == 5                   # > text capacity 16
    assert _attn([_item(L, frames=0)]) == 1
    assert _attn([_item(L, n_frames_kv=70000)]) == 5
    L8 = _layer(dtype=1)
    assert _attn([_item(L), _item(L8)]) in (2, 4)                 # mixed dtypes / fp8 P=24
    bad = _item(L)
    bad.q = FAKE + 8
    assert _attn([bad]) == 3


def test_attention_window_validation(lib):
    """Timed text windows: 8-byte alignment, video keys required when video
    rows meet text keys, and the per-workgroup table bound (255 / P + 3) *
    ceil(n_text / 32) <= 2048 words (P = 24 here: 13 rows, 157 words)."""
    def win(it, ptr):
        it.text_window = ptr
        return it
    L = _layer()
    assert _attn([win(_item(L), FAKE + 4)]) == 3
    assert _attn([win(_item(L, n_frames_kv=0), FAKE)]) == 1
    big = _layer(tc=5040)
    assert _attn([win(_item(big, n_text_kv=5025), FAKE)]) == 5
    assert b"table words" in lib.sa_last_error()
    # within the bound the item passes validation; the second item fails
    assert _attn([win(_item(big, n_text_kv=5024), FAKE), _item(L, frames=0)]) == 1
    assert b"item 1" in lib.sa_last_error()
    # windows are ignored without video rows or without text keys
    assert _attn([win(_item(L, n_text_kv=0), FAKE + 4), _item(L, frames=0)]) == 1
    assert b"item 1" in lib.sa_last_error()
    no_rows = win(_item(L, rows=False, n_frames_kv=0), FAKE + 4)
    assert _attn([no_rows]) == 0


def test_sparse_validation(lib):
    """Block-sparse history: the attention item's list fields and the
    selection call are checked on the host (P = 24: one block per frame)."""
    L = _layer(fc=8)

    def sp(it, lst=FAKE, nh=2, keep=1):
        it.block_list, it.n_hist_frames, it.keep_blocks = lst, nh, keep
        return it
    assert _attn([sp(_item(L), nh=3)]) == 5                       # n_hist_frames > n_frames_kv
    assert _attn([sp(_item(L), keep=0)]) == 1
    assert _attn([sp(_item(L), keep=3)]) == 1                     # > 2 candidates
    assert _attn([sp(_item(L), lst=FAKE + 2)]) == 3
    # ignored without candidate frames: the second item's error is reported
    assert _attn([sp(_item(L), nh=0, keep=0), _item(L, frames=0)]) == 1
    assert b"item 1" in lib.sa_last_error()
    g = _geom()
    sel = lib.sa_sparse_select
    ws = lib.sa_sparse_select_workspace
    it = sp(_item(L))
    assert ws(ctypes.byref(g), ctypes.byref(it)) == 2 * 2 * 128 * 4   # H x candidates x 128 fp32
    assert sel(ctypes.byref(g), ctypes.byref(it), ctypes.c_void_p(FAKE), 16,
               ctypes.c_void_p(FAKE), None) == 6                          # workspace too small
    assert sel(ctypes.byref(g), ctypes.byref(it), ctypes.c_void_p(FAKE), 4096, None, None) == 1
    assert sel(ctypes.byref(g), ctypes.byref(it), ctypes.c_void_p(FAKE + 4), 4096,
               ctypes.c_void_p(FAKE), None) == 3
    assert sel(ctypes.byref(g), ctypes.byref(sp(_item(L), nh=0)), ctypes.c_void_p(FAKE), 4096,
               ctypes.c_void_p(FAKE), None) == 1
    assert sel(ctypes.byref(g), ctypes.byref(sp(_item(L, rows=False))), ctypes.c_void_p(FAKE),
               4096, ctypes.c_void_p(FAKE), None) == 1                   # no query rows
    big = _layer(fc=9000)
    assert ws(ctypes.byref(g), ctypes.byref(sp(_item(big, n_frames_kv=8200), nh=8193))) == 0
    assert b"candidate blocks" in lib.sa_last_error()
    assert sel(ctypes.byref(g), None, ctypes.c_void_p(FAKE), 4096, ctypes.c_void_p(FAKE), None) == 1


def test_sparse_noalloc_validation(lib):
    """The allocation-free selection refuses, on the host, what its static
    scratch cannot hold (heads x candidates x 512 bytes > 32 MiB) and the
    block-list errors of sparse_select."""
    assert sa.SPARSE_SCRATCH_BYTES == 32 << 20
    nal = lib.sa_sparse_select_noalloc
    big = _layer(fc=5000)
    g16 = _geom(heads=16)
    it = _item(big, n_frames_kv=4097)
    it.block_list, it.n_hist_frames, it.keep_blocks = FAKE, 4097, 1     # P = 24: one block a frame
    assert nal(ctypes.byref(g16), ctypes.byref(it), ctypes.c_void_p(FAKE), None) == 6
    assert b"static scratch" in lib.sa_last_error()
    assert lib.sa_sparse_select_workspace(ctypes.byref(g16), ctypes.byref(it)) == 16 * 4097 * 512
    g = _geom()
    L = _layer(fc=8)
    it = _item(L)
    it.block_list, it.n_hist_frames, it.keep_blocks = FAKE, 2, 1
    assert nal(ctypes.byref(g), ctypes.byref(it), None, None) == 1
    assert nal(ctypes.byref(g), ctypes.byref(it), ctypes.c_void_p(FAKE + 2), None) == 3
    it.keep_blocks = 3
    assert nal(ctypes.byref(g), ctypes.byref(it), ctypes.c_void_p(FAKE), None) == 1
    assert nal(ctypes.byref(g), None, ctypes.c_void_p(FAKE), None) == 1


def test_camera_validation(lib):
    g = _geom()
    f = lib.sa_camera_attention
    ok = dict(q=FAKE, n=2, k=FAKE, v=FAKE, nc=2, hk=1, c=1, o=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(ctypes.byref(g), ctypes.c_void_p(a["q"]), a["n"], ctypes.c_void_p(a["k"]),
                 ctypes.c_void_p(a["v"]), a["nc"], a["hk"], a["c"], ctypes.c_void_p(a["o"]), None,
                 None)
    assert call(n=0) == 1
    assert call(c=0) == 1 and call(c=17) == 1
    assert call(nc=1) == 1                      # fewer camera tokens than frames
    assert call(hk=3) == 1                      # neither 1 nor H = 2
    assert call(q=0) == 1
    assert call(o=FAKE + 8) == 3


def test_attention_workspace_query_without_split(lib):
    """The workspace query launches nothing; invalid arguments (and, here, no
    device) give 0, so the call would run every tile whole."""
    L = _layer()
    g = _geom()
    q = lib.sa_segment_attention_workspace
    arr = (B.sa_attn_item * 1)(_item(L))
    assert q(ctypes.byref(g), arr, 1) == 0
    assert q(ctypes.byref(g), arr, 0) == 0
    bad = (B.sa_attn_item * 1)(_item(L, n_text_kv=17))
    assert q(ctypes.byref(g), bad, 1) == 0


def test_gather_and_dequant_validation(lib):
    g = _geom()
    src, dst = _layer(), _layer(fc=2)
    f = lib.sa_history_gather
    assert f(ctypes.byref(g), ctypes.byref(src), ctypes.c_void_p(FAKE), 3, ctypes.byref(dst), None) == 6
    assert f(ctypes.byref(g), ctypes.byref(src), None, 1, ctypes.byref(dst), None) == 1
    dst8 = _layer(dtype=1, fc=2)
    g16 = sa.Geom(heads=2, lat_h=4, lat_w=8).c()
    assert f(ctypes.byref(g16), ctypes.byref(src), ctypes.c_void_p(FAKE), 1, ctypes.byref(dst8), None) == 4
    d = lib.sa_kv_dequant
    assert d(ctypes.byref(g16), ctypes.byref(src), ctypes.c_void_p(FAKE), 1, 0, ctypes.byref(dst), None) == 4
    assert d(ctypes.byref(g16), ctypes.byref(_layer(dtype=1)), ctypes.c_void_p(FAKE), 3, 0,
             ctypes.byref(dst), None) == 6
