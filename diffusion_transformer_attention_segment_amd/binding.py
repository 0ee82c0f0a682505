"""ctypes binding of the segment-attention C ABI (include/segattn.h).

Argument marshalling only: every step of the computation runs in the HIP
library. PyTorch supplies device memory (tensor.data_ptr()) and the current
stream. If libsegattn.so has not been built, loading raises -- there is no
fallback implementation.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SEGATTN_LIBRARY may name another build of the same library (same ABI)
LIB_PATH = os.environ.get("SEGATTN_LIBRARY", os.path.join(_PKG, "libsegattn.so"))

SA_OK = 0
SA_E_ARG_STATUS = 1
STATUS_NAMES = {0: "SA_OK", 1: "SA_E_ARG", 2: "SA_E_SHAPE", 3: "SA_E_ALIGN",
                4: "SA_E_UNSUPPORTED", 5: "SA_E_RANGE", 6: "SA_E_CAPACITY", 7: "SA_E_HIP"}
KV_BF16, KV_FP8, KV_INT8 = 0, 1, 2
SEL_ALL, SEL_RECENT, SEL_POWER, SEL_ANCHOR_RECENT = 0, 1, 2, 3
MAX_ITEMS = 8
MAX_FRAMES_KV = 65536
HEAD_DIM = 128


class SegAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class sa_geom(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("lat_h", ctypes.c_int32), ("lat_w", ctypes.c_int32),
                ("rope_split", ctypes.c_int32 * 3), ("rope_theta", ctypes.c_float),
                ("softmax_scale", ctypes.c_float)]


class sa_kv_layer(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("frame_capacity", ctypes.c_int32),
                ("text_capacity", ctypes.c_int32), ("reserved0", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("k_text", ctypes.c_void_p), ("v_text", ctypes.c_void_p),
                ("k_text_scale", ctypes.c_void_p), ("v_text_scale", ctypes.c_void_p)]


class sa_attn_item(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("frame0_q", ctypes.c_int32),
                ("n_frames_q", ctypes.c_int32), ("n_text_q", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("kv", ctypes.POINTER(sa_kv_layer)),
                ("frames", ctypes.c_void_p), ("n_frames_kv", ctypes.c_int32),
                ("n_text_kv", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("text_window", ctypes.c_void_p),
                ("block_list", ctypes.c_void_p), ("n_hist_frames", ctypes.c_int32),
                ("keep_blocks", ctypes.c_int32)]


# exported symbol -> (restype, argtypes); also the list of ABI entry points
_P = ctypes.c_void_p
_I = ctypes.c_int32
SIGNATURES = {
    "sa_abi_version": (ctypes.c_int, []),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sa_cache_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_geom), _I, _I, _I]),
    "sa_kv_append": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_kv_layer), _P, _P,
                                    _I, _I, _P]),
    "sa_text_append": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_kv_layer), _P, _P,
                                      _I, _P]),
    "sa_history_select": (ctypes.c_int, [_I, _I, _I, ctypes.c_double, _I, _I,
                                         ctypes.POINTER(ctypes.c_int32), _I,
                                         ctypes.POINTER(ctypes.c_int32)]),
    "sa_history_gather": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_kv_layer), _P,
                                         _I, ctypes.POINTER(sa_kv_layer), _P]),
    "sa_segment_attention_workspace": (ctypes.c_size_t, [ctypes.POINTER(sa_geom),
                                                         ctypes.POINTER(sa_attn_item), _I]),
    "sa_segment_attention": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_attn_item),
                                            _I, _P, ctypes.c_size_t, _P]),
    "sa_segment_attention_counted": (ctypes.c_int, [ctypes.POINTER(sa_geom),
                                                    ctypes.POINTER(sa_attn_item), _I, _P,
                                                    ctypes.c_size_t, _P, _P]),
    "sa_sparse_keep": (ctypes.c_int32, [_I, _I]),
    "sa_sparse_select_workspace": (ctypes.c_size_t, [ctypes.POINTER(sa_geom),
                                                     ctypes.POINTER(sa_attn_item)]),
    "sa_sparse_select": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_attn_item), _P,
                                        ctypes.c_size_t, _P, _P]),
    "sa_sparse_select_noalloc": (ctypes.c_int, [ctypes.POINTER(sa_geom),
                                                ctypes.POINTER(sa_attn_item), _P, _P]),
    "sa_camera_attention": (ctypes.c_int, [ctypes.POINTER(sa_geom), _P, _I, _P, _P, _I, _I, _I, _P,
                                           _P, _P]),
    "sa_kv_dequant": (ctypes.c_int, [ctypes.POINTER(sa_geom), ctypes.POINTER(sa_kv_layer), _P, _I,
                                     _I, ctypes.POINTER(sa_kv_layer), _P]),
}

_lib = None


def load(path):
    """A build of the library at `path` with the C signatures set (raises if
    it is missing)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run "
                           "`python -m diffusion_transformer_attention_segment_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """The loaded library (raises if libsegattn.so is missing)."""
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


def _check(status):
    if status != SA_OK:
        raise SegAttnError(status, lib().sa_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_i32(t, n, name):
    """A device index tensor must be contiguous int32 with at least n entries."""
    if t is None:
        return
    if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name}: need a contiguous int32 tensor of at least {n} entries, "
                         f"got {t.dtype} {tuple(t.shape)}")


class Geom:
    """Attention geometry (sa_geom)."""

    def __init__(self, heads=16, lat_h=22, lat_w=40, rope_split=(16, 56, 56),
                 rope_theta=10000.0, softmax_scale=0.0, head_dim=HEAD_DIM):
        self.heads, self.lat_h, self.lat_w = heads, lat_h, lat_w
        self.rope_split = tuple(rope_split)
        self.rope_theta, self.softmax_scale, self.head_dim = rope_theta, softmax_scale, head_dim

    @property
    def P(self):
        return self.lat_h * self.lat_w

    def c(self):
        g = sa_geom()
        g.heads, g.head_dim, g.lat_h, g.lat_w = self.heads, self.head_dim, self.lat_h, self.lat_w
        for i in range(3):
            g.rope_split[i] = self.rope_split[i]
        g.rope_theta, g.softmax_scale = self.rope_theta, self.softmax_scale
        return g


def plane_slots(dtype, P):
    """Token slots of one (frame, head) plane: P for bf16, P rounded up to a
    multiple of 16 for the one-byte caches (the library's layout)."""
    return P if dtype == KV_BF16 else -(-P // 16) * 16


class KVLayer:
    """One layer's cache planes as torch tensors (caller-owned device memory)."""

    def __init__(self, dtype, k, v, k_text, v_text, k_scale=None, v_scale=None,
                 k_text_scale=None, v_text_scale=None):
        self.dtype = dtype
        self.k, self.v, self.k_text, self.v_text = k, v, k_text, v_text
        self.k_scale, self.v_scale = k_scale, v_scale
        self.k_text_scale, self.v_text_scale = k_text_scale, v_text_scale
        self.frame_capacity = k.shape[0] if k is not None else 0
        self.text_capacity = k_text.shape[1] if k_text is not None else 0
        self._c = None

    @classmethod
    def allocate(cls, geom, dtype, frame_capacity, text_capacity, device="cuda"):
        H, P, D = geom.heads, geom.P, geom.head_dim
        P = plane_slots(dtype, P)     # token slots of a frame plane
        et = {KV_BF16: torch.bfloat16, KV_FP8: torch.uint8, KV_INT8: torch.int8}[dtype]
        kw = dict(device=device, dtype=et)
        k = torch.empty((frame_capacity, H, P, D), **kw)
        v = torch.empty((frame_capacity, H, D, P), **kw)
        kt = torch.empty((H, text_capacity, D), **kw)
        vt = torch.zeros((H, D, text_capacity), **kw)
        sc = {}
        f32 = dict(device=device, dtype=torch.float32)
        if dtype == KV_FP8:
            sc = dict(k_scale=torch.ones((frame_capacity, H), **f32),
                      v_scale=torch.ones((frame_capacity, H), **f32),
                      k_text_scale=torch.ones((H,), **f32), v_text_scale=torch.ones((H,), **f32))
        elif dtype == KV_INT8:     # a scale per token and head
            sc = dict(k_scale=torch.ones((frame_capacity, H, P), **f32),
                      v_scale=torch.ones((frame_capacity, H, P), **f32),
                      k_text_scale=torch.zeros((H, text_capacity), **f32),
                      v_text_scale=torch.zeros((H, text_capacity), **f32))
        return cls(dtype, k, v, kt, vt, **sc)

    def c(self):
        if self._c is None:
            L = sa_kv_layer()
            L.dtype, L.frame_capacity, L.text_capacity = self.dtype, self.frame_capacity, self.text_capacity
            L.k, L.v = _ptr(self.k).value, _ptr(self.v).value
            L.k_text, L.v_text = _ptr(self.k_text).value, _ptr(self.v_text).value
            L.k_scale, L.v_scale = _ptr(self.k_scale).value, _ptr(self.v_scale).value
            L.k_text_scale = _ptr(self.k_text_scale).value
            L.v_text_scale = _ptr(self.v_text_scale).value
            self._c = L
        return self._c


def abi_version():
    return lib().sa_abi_version()


def last_error():
    return lib().sa_last_error().decode()


def cache_bytes(geom, dtype, frame_capacity, text_capacity):
    g = geom.c()
    n = lib().sa_cache_bytes(ctypes.byref(g), dtype, frame_capacity, text_capacity)
    if n == 0 and last_error():
        raise SegAttnError(1, last_error())
    return n


def kv_append(geom, layer, k_in, v_in, frame0, n_frames, stream=None):
    g = geom.c()
    _check(lib().sa_kv_append(ctypes.byref(g), ctypes.byref(layer.c()), _ptr(k_in), _ptr(v_in),
                              frame0, n_frames, _stream(stream)))


def text_append(geom, layer, k_in, v_in, n_text, stream=None):
    g = geom.c()
    _check(lib().sa_text_append(ctypes.byref(g), ctypes.byref(layer.c()), _ptr(k_in), _ptr(v_in),
                                n_text, _stream(stream)))


def history_select(policy, t_past, budget=0, gamma=2.0, frames_per_segment=1,
                   recent_segments=0, cap=None):
    """Host-only selection; returns a list of frame indices (ascending)."""
    if cap is None:
        cap = max(t_past, 1)
    buf = (ctypes.c_int32 * max(cap, 1))()
    n = ctypes.c_int32(0)
    _check(lib().sa_history_select(policy, t_past, budget, gamma, frames_per_segment,
                                   recent_segments, buf, cap, ctypes.byref(n)))
    return list(buf[:n.value])


def history_gather(geom, src, d_frames, n, dst, stream=None):
    g = geom.c()
    _check(lib().sa_history_gather(ctypes.byref(g), ctypes.byref(src.c()), _ptr(d_frames), n,
                                   ctypes.byref(dst.c()), _stream(stream)))


class AttnItem:
    """One session's attention call (sa_attn_item). text_window: optional
    int32 device tensor [n_text_kv, 2] of (first, last) absolute query frames
    that see each text key. block_list: optional int32 device tensor
    [H, ceil(rows / 256), keep_blocks] of kept history blocks over the first
    n_hist_frames frames (block-sparse history; sparse_select writes it)."""

    def __init__(self, q, layer, frames, n_frames_kv, n_text_kv, out, frame0_q, n_frames_q,
                 n_text_q, lse=None, text_window=None, block_list=None, n_hist_frames=0,
                 keep_blocks=0):
        self.q, self.layer, self.frames, self.out, self.lse = q, layer, frames, out, lse
        self.text_window = text_window
        self.block_list, self.n_hist_frames, self.keep_blocks = block_list, n_hist_frames, keep_blocks
        self.n_frames_kv, self.n_text_kv = n_frames_kv, n_text_kv
        self.frame0_q, self.n_frames_q, self.n_text_q = frame0_q, n_frames_q, n_text_q

    def c(self):
        _check_i32(self.frames, self.n_frames_kv, "frames")
        _check_i32(self.text_window, 2 * self.n_text_kv, "text_window")
        _check_i32(self.block_list, self.keep_blocks, "block_list")
        it = sa_attn_item()
        it.q = _ptr(self.q).value
        it.frame0_q, it.n_frames_q, it.n_text_q = self.frame0_q, self.n_frames_q, self.n_text_q
        it.kv = ctypes.pointer(self.layer.c())
        it.frames = _ptr(self.frames).value
        it.n_frames_kv, it.n_text_kv = self.n_frames_kv, self.n_text_kv
        it.out = _ptr(self.out).value
        it.lse = _ptr(self.lse).value
        it.text_window = _ptr(self.text_window).value
        it.block_list = _ptr(self.block_list).value
        it.n_hist_frames, it.keep_blocks = self.n_hist_frames, self.keep_blocks
        return it


def segment_attention_workspace(geom, items):
    """Bytes of device workspace the split plan of this call wants (0: none)."""
    g = geom.c()
    arr = (sa_attn_item * max(len(items), 1))()
    for i, it in enumerate(items):
        arr[i] = it.c()
    return int(lib().sa_segment_attention_workspace(ctypes.byref(g), arr, len(items)))


def segment_attention(geom, items, stream=None, workspace="auto", counters=None):
    """Joint segment attention over the items.

    workspace: "auto" allocates what sa_segment_attention_workspace asks for
    (the last round's tiles are then split over key ranges and merged); None
    runs every tile whole; a uint8 CUDA tensor is used as given (too small:
    whole tiles). counters: an int32 CUDA tensor of >= 3 entries runs
    sa_segment_attention_counted, which adds [work tiles, slow-path events,
    rescale steps] into it (same outputs)."""
    g = geom.c()
    arr = (sa_attn_item * max(len(items), 1))()
    for i, it in enumerate(items):
        arr[i] = it.c()
    ws, nbytes = None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError(f"workspace must be 'auto', None or a tensor, not {workspace!r}")
        nbytes = int(lib().sa_segment_attention_workspace(ctypes.byref(g), arr, len(items)))
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=items[0].q.device)
            if stream is not None:
                ext = stream if isinstance(stream, torch.cuda.Stream) else \
                    torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
                ws.record_stream(ext)
    elif workspace is not None:
        ws, nbytes = workspace, workspace.numel() * workspace.element_size()
    if counters is not None:
        _check_i32(counters, 3, "counters")
        _check(lib().sa_segment_attention_counted(ctypes.byref(g), arr, len(items), _ptr(ws),
                                                  nbytes, _ptr(counters), _stream(stream)))
        return
    _check(lib().sa_segment_attention(ctypes.byref(g), arr, len(items), _ptr(ws), nbytes,
                                      _stream(stream)))


SPARSE_KEY_BLOCK, SPARSE_QUERY_BLOCK = 64, 256


def sparse_keep(n_candidates, percent):
    """Blocks kept out of n_candidates at `percent` (the library's rule:
    ceil, at least 1, at most all)."""
    n = lib().sa_sparse_keep(int(n_candidates), int(percent))
    if n < 0:
        _check(SA_E_ARG_STATUS)
    return int(n)


def sparse_select(geom, item, block_list=None, stream=None):
    """Block lists of the item (its n_hist_frames and keep_blocks) for
    block-sparse history attention: int32 [H, ceil(rows / 256), keep_blocks]
    (allocated when block_list is None). The pooled-key workspace is
    allocated through torch."""
    g = geom.c()
    it = item.c()
    nbytes = int(lib().sa_sparse_select_workspace(ctypes.byref(g), ctypes.byref(it)))
    rows = item.n_frames_q * geom.P + item.n_text_q
    if block_list is None:
        nq = -(-rows // SPARSE_QUERY_BLOCK)
        block_list = torch.empty((geom.heads, max(nq, 1), max(item.keep_blocks, 1)),
                                 dtype=torch.int32, device=item.q.device)
    else:
        _check_i32(block_list, geom.heads * -(-rows // SPARSE_QUERY_BLOCK) * item.keep_blocks,
                   "block_list")
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=item.q.device)
    _check(lib().sa_sparse_select(ctypes.byref(g), ctypes.byref(it), _ptr(ws), nbytes,
                                  _ptr(block_list), _stream(stream)))
    if stream is not None:
        ext = stream if isinstance(stream, torch.cuda.Stream) else \
            torch.cuda.ExternalStream(int(getattr(stream, "cuda_stream", stream)))
        ws.record_stream(ext)
    return block_list


SPARSE_SCRATCH_BYTES = 32 << 20


def sparse_select_noalloc(geom, item, block_list, stream=None):
    """sparse_select with the pooled keys in the library's static device
    scratch (SPARSE_SCRATCH_BYTES per GPU): the call allocates nothing, so
    block_list (int32 [H, ceil(rows / 256), keep_blocks], device) is the
    caller's. Calls that overlap in time on one GPU share the scratch and
    race."""
    rows = item.n_frames_q * geom.P + item.n_text_q
    _check_i32(block_list, geom.heads * -(-rows // SPARSE_QUERY_BLOCK) * item.keep_blocks,
               "block_list")
    g = geom.c()
    it = item.c()
    _check(lib().sa_sparse_select_noalloc(ctypes.byref(g), ctypes.byref(it), _ptr(block_list),
                                          _stream(stream)))
    return block_list


MAX_CAMERA_CHUNK = 16


def camera_attention(geom, q, n_frames, cam_k, cam_v, chunk, out, lse=None, stream=None):
    """Cross-attention of the video queries q [n_frames * P, H, 128] to the
    camera tokens cam_k, cam_v [n_cam, kv_heads, 128] (kv_heads 1 or H):
    latent frame t sees the tokens of its chunk of `chunk` frames."""
    g = geom.c()
    _check(lib().sa_camera_attention(ctypes.byref(g), _ptr(q), n_frames, _ptr(cam_k), _ptr(cam_v),
                                     cam_k.shape[0], cam_k.shape[1], chunk, _ptr(out), _ptr(lse),
                                     _stream(stream)))


def kv_dequant(geom, src, d_frames, n_frames, n_text, dst, stream=None):
    g = geom.c()
    _check(lib().sa_kv_dequant(ctypes.byref(g), ctypes.byref(src.c()), _ptr(d_frames), n_frames,
                               n_text, ctypes.byref(dst.c()), _stream(stream)))
