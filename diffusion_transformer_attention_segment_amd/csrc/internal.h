// Internal declarations shared by the host layer and the HIP kernel files.
// Not part of the public ABI (include/segattn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/segattn.h"

namespace segattn {

constexpr int kD = SA_HEAD_DIM;   // head dim (128)

// Per-call RoPE description shared by the append and attention kernels.
struct RopeParams {
  int32_t split0, split1, split2;  // t, h, w band widths (even, sum 128)
  int32_t lat_w;                   // tokens per latent row
  int32_t P;                       // tokens per latent frame
  double log2_theta;               // log2(theta), for the fp64 frequencies
};

// ---- kv_append / text_append ------------------------------------------------
// Token slots of one (frame, head) plane: P, rounded up to a multiple of 16
// for the one-byte caches (e4m3, int8) so that every V^T row starts 16-byte
// aligned. Slots past P hold zero V^T codes (and zero int8 scales); K rows
// past P are never read.
__host__ __device__ inline int plane_tokens(int P, bool one_byte) {
  return one_byte ? (P + 15) & ~15 : P;
}

struct AppendArgs {
  const uint16_t* k_in;     // bf16 [n_tokens][H][128]
  const uint16_t* v_in;
  void* k;                  // plane base (frame 0 / text slot base)
  void* v;
  float* k_scale;           // fp8: [frames][H] or [H] for text; int8: [frames][H][P] or [H][cap]
  float* v_scale;
  int32_t heads;
  int32_t frame0;           // first frame written (video); unused for text
  int32_t n_frames;         // video frames (video) / 1 (text)
  int32_t plane_len;        // P for video, text_capacity for text
  int32_t n_tok;            // valid tokens per plane (P for video, n_text)
  int32_t is_text;          // 1: text slot (no rotation, zero-fill V tail)
  RopeParams rope;
};

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_fp8(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_int8(const AppendArgs& a, hipStream_t s);

// ---- attention ----------------------------------------------------------------
struct AttnItemDev {
  const uint16_t* q;
  uint16_t* out;
  float* lse;
  const void* k;
  const void* v;
  const void* k_text;
  const void* v_text;
  const float* k_scale;
  const float* v_scale;
  const float* k_text_scale;
  const float* v_text_scale;
  const int32_t* frames;
  int32_t frame0_q;
  int32_t n_q_video;     // video query rows
  int32_t n_q;           // all query rows (video + text)
  int32_t n_frames_kv;
  int32_t n_text_kv;
  int32_t text_cap;
  const int32_t* text_window;   // [n_text_kv][2] (first, last) frames, or NULL: no windows
  const int32_t* block_list;    // [H][q_tiles][keep] kept history tiles, or NULL: dense
  int32_t n_hist_frames;        // candidate frames (first entries of `frames`) when sparse
  int32_t keep;                 // list length when sparse
  int32_t q_tiles;       // ceil(n_q / BLOCK_M)
  int32_t tile_begin;    // first logical tile of this item (over heads * q_tiles)
};

// Work: total_tiles logical query tiles ordered (item, head, query tile). The
// first n_full run whole; each later one runs as split_k parts over its key
// tiles (part p: [p n / split_k, (p+1) n / split_k)), writing partials to ws:
// for unit u = (tile - n_full) * split_k + part, O [BM][128] at
// ws + u * BM * kPartialStride, then m [BM] and l [BM] (log2-unit max and sum
// of the exponentials against it; O is not normalised).
struct AttnArgs {
  AttnItemDev items[SA_MAX_ITEMS];
  int32_t n_items;
  int32_t heads;
  int32_t total_tiles;
  int32_t n_full;
  int32_t split_k;        // 1: nothing is split
  int32_t grid;           // n_full + (total_tiles - n_full) * split_k
  int32_t any_sparse;     // 1: some item has a block list (the sparse kernel instantiation)
  int32_t int8;           // 1: int8 layers (the bf16 kernel dequantises while staging tiles)
  float* ws;
  float scale_log2;       // softmax scale * log2(e)
  RopeParams rope;
  uint32_t* counters;     // optional diagnostics (NULL: none), see add_counts
};

constexpr int kPartialStride = kD + 2;   // floats per row of a partial: O, m, l

// Timed text windows reach the kernels as a per-workgroup visibility table in
// LDS: one bit per text key (bit b of word w: key 32 w + b), row 0 all ones
// (text query rows), then one row per latent frame that the workgroup's video
// query rows span, in frame order. A workgroup of block_m rows spans at most
// (block_m - 1) / P + 2 frames of P tokens.
constexpr int kWindowWords = SA_WINDOW_TABLE_WORDS;   // table capacity (words)
__host__ __device__ inline int window_row_words(int n_text) { return (n_text + 31) / 32; }
__host__ __device__ inline int window_table_rows(int P, int block_m) { return (block_m - 1) / P + 3; }

// ---- sparse history: block selection -------------------------------------------
// pool_k: mean stored key of every candidate block, fp32 [H][128][n_cand].
// select: per (head, query block) the keep best blocks by pooled q . pooled k.
struct SelectArgs {
  AttnItemDev item;        // q, kv planes, frames, counts of the session
  int32_t heads;
  int32_t fp8;             // 1: e4m3 planes with per-(frame, head) scales
  int32_t int8;            // 1: int8 planes with per-token scales
  int32_t n_cand;          // n_hist_frames * ceil(P / 64)
  int32_t keep;
  float* pooled;           // workspace [H][128][n_cand]
  int32_t* out;            // [H][q_tiles][keep]
  RopeParams rope;
};
constexpr int kMaxCandidates = SA_MAX_SPARSE_CANDIDATES;
hipError_t launch_sparse_select(const SelectArgs& a, hipStream_t s);
// Device address of the static pooled-key array (SA_SPARSE_SCRATCH_BYTES) on
// the current device, looked up on the first call per device.
hipError_t sparse_select_scratch(float** out);

hipError_t launch_attention_bf16(AttnArgs& a, hipStream_t s);
hipError_t launch_attention_fp8(AttnArgs& a, hipStream_t s);
hipError_t launch_attention_combine(const AttnArgs& a, int block_m, hipStream_t s);
int attention_block_m_bf16();
int attention_block_m_fp8();

// ---- camera cross-attention ------------------------------------------------------
struct CameraArgs {
  const uint16_t* q;       // bf16 [rows][H][128]
  const uint16_t* cam_k;   // bf16 [n_cam][kv_heads][128]
  const uint16_t* cam_v;
  uint16_t* out;           // bf16 [rows][H][128]
  float* lse;              // optional fp32 [rows][H]
  int32_t rows;            // n_frames * P
  int32_t heads;
  int32_t kv_heads;        // 1 or heads
  int32_t P;
  int32_t n_cam;
  int32_t chunk;
  float scale_log2;        // softmax scale * log2(e)
};
hipError_t launch_camera(const CameraArgs& a, hipStream_t s);

// ---- gather / dequant -----------------------------------------------------------
struct GatherArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const float* src_ks;
  const float* src_vs;
  float* dst_ks;
  float* dst_vs;
  const int32_t* frames;
  int32_t n;
  int64_t plane_bytes;     // bytes of one frame's K (= V) plane over all heads
  int64_t scale_floats;    // scales per frame (fp8: H, int8: H * P); 0 for bf16
  int32_t heads;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t s);

struct DequantArgs {
  const uint8_t* src_k;    // fp8 or int8 plane base
  const uint8_t* src_v;
  const float* src_ks;     // [frames][H] or [H]
  const float* src_vs;
  uint16_t* dst_k;         // bf16 plane base
  uint16_t* dst_v;
  const int32_t* frames;   // NULL for the text slot
  int32_t n;               // frames (or 1 for text)
  int32_t heads;
  int32_t src_len;         // tokens per source plane (P or text_capacity)
  int32_t dst_len;         // tokens per destination plane
  int32_t n_tok;           // tokens to convert per plane
  int32_t int8;            // 1: int8 codes with per-token scales (src_ks/src_vs [planes][src_len])
};
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);

}  // namespace segattn
