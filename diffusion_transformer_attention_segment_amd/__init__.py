"""Segment attention for a segment-autoregressive MMDiT world model, on MI355X.

A HIP library for gfx950 (libsegattn.so, C ABI in include/segattn.h) plus this
thin ctypes binding. The calls follow the method's hot path:

* ``history_select``  -- host-only pick of the kept past frames
* ``history_gather``  -- materialise picked frames into a compact buffer
* ``kv_append`` / ``text_append`` -- fused 3D RoPE + cache write (bf16 / e4m3 / int8)
* ``segment_attention`` -- Q-RoPE, Q.K^T, online softmax, .V over
  [kept frames ; own segment ; own text], gather-fused
* ``sparse_select``   -- block lists for block-sparse history attention
  (``sparse_select_noalloc``: the same, with no allocation in the call)
* ``camera_attention`` -- video tokens to their frame chunk's camera tokens
* ``kv_dequant``      -- e4m3 or int8 cache -> bf16 planes
"""

from .binding import (  # noqa: F401
    AttnItem, Geom, KVLayer, SegAttnError, MAX_CAMERA_CHUNK, camera_attention, KV_BF16, KV_FP8,
    KV_INT8, SEL_ALL, SEL_RECENT, SEL_POWER,
    SEL_ANCHOR_RECENT, MAX_ITEMS, MAX_FRAMES_KV, HEAD_DIM, SIGNATURES, LIB_PATH, abi_version,
    cache_bytes,
    history_gather, history_select, kv_append, kv_dequant, last_error, lib, segment_attention,
    segment_attention_workspace, sparse_keep, sparse_select, sparse_select_noalloc,
    SPARSE_SCRATCH_BYTES, SPARSE_KEY_BLOCK, SPARSE_QUERY_BLOCK,
    text_append,
)
