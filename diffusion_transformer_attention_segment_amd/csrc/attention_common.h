// Pieces shared by the bf16 and fp8 segment-attention kernels: the
// workgroup -> (session, head, query tile) mapping, the scalar walk over a
// session's key tiles, and small cross-lane helpers.
#pragma once

#include "device_common.h"

namespace segattn {

constexpr int kKeyTile = 64;               // keys per tile (both kernels)
constexpr int kRsrcFlags = 0x00020000;     // raw buffer resource, 32-bit data format

// Workgroups go round-robin over the 8 XCDs. The whole tiles (the first
// n_full logical tiles) are remapped so that each XCD gets a contiguous run of
// them (same head => shared K/V in that XCD's L2); logical tiles are ordered
// (item, head, query tile). The split units that follow (the last tiles, each
// as split_k key-range parts) keep dispatch order, so they spread over every
// XCD and fill the CUs that finish their whole tiles first.
struct WorkTile {
  int item;
  int head;
  int q0;
  int part;     // key-range part of a split tile, or -1 (whole tile)
  int unit;     // partial-result slot of a split tile
};

__device__ __forceinline__ WorkTile map_workgroup(const AttnArgs& a, int block_m) {
  const int b = blockIdx.x;
  int logical;
  WorkTile w;
  if (b < a.n_full) {
    const int nb = a.n_full;
    const int xcd = b & 7, idx = b >> 3;
    const int per = nb >> 3, rem = nb & 7;
    logical = xcd * per + min(xcd, rem) + idx;   // XCD x: per + (x < rem) tiles
    w.part = -1;
    w.unit = 0;
  } else {
    // split parts, dispatched part-major: the workgroups an XCD runs at the
    // same time hold the same key range of many tiles, which then share one
    // pass of it through the XCD's L2
    const int bp = b - a.n_full;
    const int r = (a.grid - a.n_full) / a.split_k;   // split tiles
    w.part = bp / r;
    const int tile = bp - w.part * r;
    logical = a.n_full + tile;
    w.unit = tile * a.split_k + w.part;                // partial slot: parts of a tile together
  }
  int it = 0;
#pragma unroll 1
  for (int j = 1; j < a.n_items; ++j)
    if (logical >= a.items[j].tile_begin) it = j;
  const AttnItemDev& I = a.items[it];
  const int local = logical - I.tile_begin;
  w.item = it;
  w.head = local / I.q_tiles;
  w.q0 = (local - w.head * I.q_tiles) * block_m;
  return w;
}

// Scalar walk over the key tiles of one (item, head): video frames in list
// order (ceil(P / 64) tiles each, never straddling a frame), then the text
// slot. Everything here is wave-uniform. ESZ is the cache kind (below).
// Frame-list entries are read with scalar loads through the constant address
// space (the list is written before the launch and never during it).
typedef const __attribute__((address_space(4))) int* const_int_ptr;

__device__ __forceinline__ int frame_entry(const AttnItemDev& I, int fi) {
  return reinterpret_cast<const_int_ptr>(reinterpret_cast<uintptr_t>(I.frames))[fi];
}

// The same for the fp32 plane scales (written before the launch).
typedef const __attribute__((address_space(4))) float* const_float_ptr;

__device__ __forceinline__ float scalar_load(const float* p, size_t i) {
  return reinterpret_cast<const_float_ptr>(reinterpret_cast<uintptr_t>(p))[i];
}

struct TileCursor {
  int fi;               // segment: frame-list index, or n_frames (the text slot)
  int fnext;            // frame-list entry fi (before entering it), prefetched
  int p0;               // first key of the tile within its segment
  int len;              // keys in the segment (P or n_text)
  const char* kplane;   // K plane of the segment
  const char* vplane;   // V^T plane of the segment
  int vstride;          // tokens per V^T row of the plane (P or text capacity)
  float kscale;         // fp8 planes: the segment's K and V scales (1 for bf16)
  float vscale;
  const float* kst;     // int8 planes: the segment's per-token K and V scales
  const float* vst;
};

// Cache kinds, the template argument ESZ of the key-tile walk: bf16 (2 bytes
// an element), e4m3 with a scale per (frame, head) plane (1 byte), int8 with a
// scale per token and head (1 byte).
constexpr int kCkBf16 = 2, kCkFp8 = 1, kCkInt8 = 3;
template <int ESZ>
__device__ __forceinline__ constexpr int elem_bytes() {
  return ESZ == kCkBf16 ? 2 : 1;
}

template <int ESZ>
__device__ __forceinline__ void cursor_enter(TileCursor& c, const AttnItemDev& I, int h, int H,
                                             int P) {
  c.p0 = 0;
  c.kscale = 1.0f;
  c.vscale = 1.0f;
  if (c.fi < I.n_frames_kv) {
    const int frame = c.fnext;
    if (c.fi + 1 < I.n_frames_kv) c.fnext = frame_entry(I, c.fi + 1);   // one frame ahead
    const size_t pl = static_cast<size_t>(frame) * H + h;
    const int PL = plane_tokens(P, ESZ != kCkBf16);   // token slots of the plane
    const size_t plane = pl * static_cast<size_t>(PL) * kD * elem_bytes<ESZ>();
    c.kplane = static_cast<const char*>(I.k) + plane;
    c.vplane = static_cast<const char*>(I.v) + plane;
    c.len = P;
    c.vstride = PL;
    if (ESZ == kCkFp8) {
      c.kscale = scalar_load(I.k_scale, pl);
      c.vscale = scalar_load(I.v_scale, pl);
    }
    if (ESZ == kCkInt8) {
      c.kst = I.k_scale + pl * PL;
      c.vst = I.v_scale + pl * PL;
    }
  } else {
    const size_t plane = static_cast<size_t>(h) * I.text_cap * kD * elem_bytes<ESZ>();
    c.kplane = static_cast<const char*>(I.k_text) + plane;
    c.vplane = static_cast<const char*>(I.v_text) + plane;
    c.len = I.n_text_kv;
    c.vstride = I.text_cap;
    if (ESZ == kCkFp8 && I.n_text_kv > 0) {
      c.kscale = scalar_load(I.k_text_scale, h);
      c.vscale = scalar_load(I.v_text_scale, h);
    }
    if (ESZ == kCkInt8) {
      c.kst = I.k_text_scale + static_cast<size_t>(h) * I.text_cap;
      c.vst = I.v_text_scale + static_cast<size_t>(h) * I.text_cap;
    }
  }
}

// Cursor at key tile `tile` of the item (frames in list order, ceil(P / 64)
// tiles each, then the text slot).
template <int ESZ>
__device__ __forceinline__ void cursor_start(TileCursor& c, const AttnItemDev& I, int h, int H,
                                             int P, int tile = 0) {
  const int tpf = (P + kKeyTile - 1) / kKeyTile;
  const int nvid = I.n_frames_kv * tpf;
  c.fi = tile < nvid ? tile / tpf : I.n_frames_kv;
  c.fnext = c.fi < I.n_frames_kv ? frame_entry(I, c.fi) : 0;
  cursor_enter<ESZ>(c, I, h, H, P);
  c.p0 = (tile < nvid ? tile - c.fi * tpf : tile - nvid) * kKeyTile;
}

// Cursor to the next key tile of the item.
template <int ESZ>
__device__ __forceinline__ void cursor_next(TileCursor& c, const AttnItemDev& I, int h, int H,
                                            int P) {
  c.p0 += kKeyTile;
  if (c.p0 >= c.len) {
    ++c.fi;
    if (c.fi <= I.n_frames_kv) cursor_enter<ESZ>(c, I, h, H, P);
  }
}

// Key-tile sequence of a work tile, over logical index li. Dense: the item's
// tiles in order. Block-sparse history: first the kept candidate tiles of
// this (head, query tile), read from its block list, then every tile after the
// history (the remaining frames, then the text slot).
struct TileSeq {
  const int32_t* list;   // this work tile's kept tiles, or nullptr (dense)
  int keep;              // list length (0: dense)
  int after;             // first tile after the history
};

__device__ __forceinline__ TileSeq tile_seq(const AttnItemDev& I, int h, int q0, int block_m,
                                            int P) {
  TileSeq s{nullptr, 0, 0};
  if (I.block_list != nullptr) {
    const int qt = q0 / block_m;
    s.list = I.block_list + (static_cast<size_t>(h) * I.q_tiles + qt) * I.keep;
    s.keep = I.keep;
    s.after = I.n_hist_frames * ((P + kKeyTile - 1) / kKeyTile);
  }
  return s;
}

// tiles of the text slot, and logical tiles before it
__device__ __forceinline__ int text_tiles(const AttnItemDev& I) {
  return (I.n_text_kv + kKeyTile - 1) / kKeyTile;
}
__device__ __forceinline__ int seq_video_tiles(const AttnItemDev& I, int P) {
  const int tpf = (P + kKeyTile - 1) / kKeyTile;
  return I.block_list != nullptr ? I.keep + (I.n_frames_kv - I.n_hist_frames) * tpf
                                 : I.n_frames_kv * tpf;
}

// item tile of logical tile li (block-list entries read by scalar loads; the
// list is written before the launch)
__device__ __forceinline__ int seq_tile(const TileSeq& s, int li) {
  if (s.list == nullptr) return li;
  return li < s.keep ? reinterpret_cast<const_int_ptr>(reinterpret_cast<uintptr_t>(s.list))[li]
                     : s.after + li - s.keep;
}

// The kernels come in a dense and a sparse instantiation (kSparse), launched
// for calls without and with block lists: the dense walk keeps the plain
// cursor steps.
template <bool kSparse, int ESZ>
__device__ __forceinline__ void seq_start(TileCursor& c, const AttnItemDev& I, int h, int H, int P,
                                          const TileSeq& s, int li) {
  cursor_start<ESZ>(c, I, h, H, P, kSparse ? seq_tile(s, li) : li);
}

// Move the cursor on to logical tile li (the one after its current tile): a
// jump while in the kept list and onto the first tile after it, a step after.
template <bool kSparse, int ESZ>
__device__ __forceinline__ void seq_next(TileCursor& c, const AttnItemDev& I, int h, int H, int P,
                                         const TileSeq& s, int li) {
  if (kSparse && li <= s.keep)   // (never for a dense item: keep 0, li >= 1)
    cursor_start<ESZ>(c, I, h, H, P, seq_tile(s, li));
  else
    cursor_next<ESZ>(c, I, h, H, P);
}

// Logical key tiles [begin, end) of a work tile: all of them, or part `part`
// of split_k.
__device__ __forceinline__ void key_range(const AttnArgs& a, const AttnItemDev& I, int P, int part,
                                          int* begin, int* end) {
  const int n = seq_video_tiles(I, P) + text_tiles(I);
  if (part < 0) {
    *begin = 0;
    *end = n;
  } else {
    // with timed text windows the parts divide the video tiles (at least one
    // each) and the last part takes the text tiles as well: every part then
    // starts with a tile whose valid keys every query row sees
    const int ns = I.text_window != nullptr ? seq_video_tiles(I, P) : n;
    *begin = static_cast<int>(static_cast<int64_t>(part) * ns / a.split_k);
    *end = part + 1 == a.split_k ? n
                                 : static_cast<int>(static_cast<int64_t>(part + 1) * ns / a.split_k);
  }
}

// Partial result of one row of a split tile: unnormalised O (128 floats, the
// lane's 64 in MFMA output order: dims 32 db + 8 r4 + 4 g .. +3 hold
// o[db][4 r4 .. 4 r4 + 3]), then (lane half 0) m and l.
// Diagnostic counters of sa_segment_attention_counted, added once per wave
// after its key loop: [0] work tiles run, [1] slow-path events (bf16: a work
// tile whose key loop ran again with rescaling; fp8: a wave's renormalisation
// of O), [2] rescale steps of waves. Device-scope integer adds: the totals do
// not depend on their order.
__device__ __forceinline__ void add_counts(uint32_t* c, int tid, uint32_t wave_slow,
                                           uint32_t wave_rescales) {
  if ((tid & 63) != 0) return;
  if (tid == 0) atomicAdd(c, 1u);
  if (wave_slow != 0) atomicAdd(c + 1, wave_slow);
  if (wave_rescales != 0) atomicAdd(c + 2, wave_rescales);
}

__device__ __forceinline__ void store_partial(const AttnArgs& a, int unit, int block_m, int row,
                                              int g, const f32x16* o, float scale, float m,
                                              float l) {
  float* base = a.ws + static_cast<size_t>(unit) * block_m * kPartialStride;
  float* orow = base + static_cast<size_t>(row) * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 v;
      v.x = o[db][4 * r4] * scale;
      v.y = o[db][4 * r4 + 1] * scale;
      v.z = o[db][4 * r4 + 2] * scale;
      v.w = o[db][4 * r4 + 3] * scale;
      *reinterpret_cast<float4*>(orow + 32 * db + 8 * r4 + 4 * g) = v;
    }
  if (g == 0) {
    base[static_cast<size_t>(block_m) * kD + row] = m;
    base[static_cast<size_t>(block_m) * (kD + 1) + row] = l;
  }
}

__device__ __forceinline__ int cursor_nvalid(const TileCursor& c) {
  return min(kKeyTile, c.len - c.p0);
}

// Valid-key count of the cursor's tile, with the sign bit set when the tile
// holds text keys under timed text windows: one signed compare against the
// tile size then sends partial tiles and windowed text tiles alike to the
// (rare) masking path. tile_count() takes the count back out. flag_fi is the
// first segment whose tiles carry the flag (window_flag_segment), kept in a
// register so that the per-tile code reads nothing from memory.
constexpr int kWindowFlag = static_cast<int>(0x80000000u);
__device__ __forceinline__ int window_flag_segment(const AttnItemDev& I) {
  return __builtin_amdgcn_readfirstlane(I.text_window != nullptr ? I.n_frames_kv : 0x7fffffff);
}
__device__ __forceinline__ int cursor_mask_code(const TileCursor& c, int flag_fi) {
  const int n = cursor_nvalid(c);
  return c.fi >= flag_fi ? (n | kWindowFlag) : n;
}
__device__ __forceinline__ int tile_count(int code) { return code & ~kWindowFlag; }

// Buffer resources of the cursor's tile: the K resource covers the tile's
// valid rows (rows past them read as zero), the V^T resource runs from the
// tile's first column to the plane end (so no read leaves the plane).
template <int ESZ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_k_rsrc(const TileCursor& c) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(c.kplane + static_cast<size_t>(c.p0) * kD * elem_bytes<ESZ>()),
      static_cast<short>(0), cursor_nvalid(c) * kD * elem_bytes<ESZ>(), kRsrcFlags);
}

template <int ESZ>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_v_rsrc(const TileCursor& c) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.vplane + c.p0 * elem_bytes<ESZ>()),
                                           static_cast<short>(0),
                                           (c.vstride * kD - c.p0) * elem_bytes<ESZ>(), kRsrcFlags);
}

// int8 planes: the per-token K / V scales of the tile's valid keys (scales of
// keys past the valid count read as zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_scale_rsrc(const float* st,
                                                                 const TileCursor& c) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(st + c.p0), static_cast<short>(0),
                                           cursor_nvalid(c) * 4, kRsrcFlags);
}

// Direct-to-LDS tile loads. A stage is ROWS rows of SLOTS 16-byte slots (the
// last slot of each row is padding); buffer loads with the LDS flag write lane
// L's 16 bytes to the load's LDS base + 16 L (lanes whose offset is out of the
// resource write zeros), so load j fills slots 64 j .. 64 j + 63. Wave w of an
// 8-wave workgroup issues loads j = w, w + 8, ... The global offset of slot
// (row, ch) is row * row_bytes + 16 ch; padding slots load out of range.
// Returns the number of loads this wave issued.
constexpr uint32_t kOutOfRange = 0x80000000u;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The lane's index in its wave, recomputed (mbcnt) where it is used: as
// volatile asm it is not hoisted out of a loop, so neither it nor the
// per-lane values derived from it occupy a register across the loop.
__device__ __forceinline__ uint32_t lane_here() {
  uint32_t lane;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n v_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  return lane;
}

template <int ROWS, int SLOTS>
__device__ __forceinline__ int dma_tile(__amdgpu_buffer_rsrc_t r, void* stage, uint32_t row_bytes,
                                        int w) {
  constexpr int kLoads = ROWS * SLOTS / 64;
  static_assert(ROWS * SLOTS % 64 == 0, "a stage is a whole number of 1 KB loads");
  const uint32_t lane = lane_here();   // per tile: no per-lane offsets kept across the loop
  int n_issued = 0;
#pragma unroll
  for (int m = 0; m < (kLoads + 7) / 8; ++m) {
    const int j = w + 8 * m;
    if (j < kLoads) {
      const uint32_t n = 64u * j + lane;
      const uint32_t row = n / SLOTS, ch = n - SLOTS * row;
      const uint32_t off = ch == SLOTS - 1 ? kOutOfRange : row * row_bytes + ch * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_ptr_t)(static_cast<char*>(stage) + 1024 * j), 16, off, 0, 0, 0);
      ++n_issued;
    }
  }
  return n_issued;
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (n rounded down to 0, 1, 2 or 4).
__device__ __forceinline__ void wait_loads(int n) {
  if (n >= 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
  else if (n >= 2)
    __builtin_amdgcn_s_waitcnt(0x0F72);   // vmcnt(2)
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(0x0F71);   // vmcnt(1)
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
}

// max(x, x of the lane 32 away): both halves of a wave end with the same value.
__device__ __forceinline__ float max_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// ---- timed text windows -------------------------------------------------------
// Optional per item ("How one segment is made", the second mask: an action's
// text is hidden from video frames outside its time window): text key j is visible to a video
// query of absolute frame t only if window[j].x <= t <= window[j].y; text
// queries see every key. Each workgroup turns the windows into its bit table
// (layout next to kWindowWords) before its first barrier.
__device__ __forceinline__ void stage_window_table(const AttnItemDev& I, uint32_t* tab, int q0,
                                                   int bm, int P, int tid, int nthreads) {
  if (I.text_window == nullptr) return;
  const int words = window_row_words(I.n_text_kv);
  const int last = min(q0 + bm, I.n_q_video) - 1;   // last video row of the workgroup
  const int fa = q0 / P;
  const int rows = 1 + (last >= q0 ? last / P - fa + 1 : 0);
  const int2* win = reinterpret_cast<const int2*>(I.text_window);
  for (int e = tid; e < rows * words; e += nthreads) {
    const int row = e / words, w = e - row * words;
    uint32_t bits = ~0u;
    if (row > 0) {
      const int t = I.frame0_q + fa + row - 1;
      const int nb = min(32, I.n_text_kv - 32 * w);
      bits = 0u;
      for (int b = 0; b < nb; ++b) {
        const int2 wj = win[32 * w + b];
        bits |= static_cast<uint32_t>(wj.x <= t && t <= wj.y) << b;
      }
    }
    tab[e] = bits;
  }
}

// word offset of query row `row`'s table row (0, all visible, for text rows)
__device__ __forceinline__ int window_row_offset(const AttnItemDev& I, int q0, int row, int P) {
  if (I.text_window == nullptr || row >= I.n_q_video) return 0;
  return (row / P - q0 / P + 1) * window_row_words(I.n_text_kv);
}

// text index of the first key of logical text tile `tile` (text comes last)
__device__ __forceinline__ int text_tile_base(const AttnItemDev& I, int P, int tile) {
  return (tile - seq_video_tiles(I, P)) * kKeyTile;
}

// s if bit `bit` of `word` is set, else -inf (bit-field insert under a
// sign-extended one-bit mask)
__device__ __forceinline__ float keep_if_bit(float s, uint32_t word, int bit) {
  const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(word << (31 - bit)) >> 31);
  return __uint_as_float((__float_as_uint(s) & m) | (0xFF800000u & ~m));
}

// RoPE position of query row `row` (video rows in raster order, then text).
__device__ __forceinline__ void query_position(const AttnItemDev& I, const RopeParams& r, int row,
                                               bool* video, int* t, int* hh, int* ww) {
  *video = row < I.n_q_video;
  *t = *hh = *ww = 0;
  if (*video) {
    const int f = row / r.P, p = row - (row / r.P) * r.P;
    *t = I.frame0_q + f;
    *hh = p / r.lat_w;
    *ww = p - *hh * r.lat_w;
  }
}

}  // namespace segattn
