/*
 * segattn.h -- C ABI of the segment-attention library (HIP, gfx950 / MI355X).
 *
 * What it computes. In a segment-autoregressive MMDiT world model, the joint
 * attention of each dual-stream block takes as queries the current segment's
 * latent video tokens followed by its text tokens, and as keys/values the
 * per-layer KV cache of earlier segments plus the segment itself, with no mask
 * inside the segment (optionally, timed text windows hide text keys from
 * video queries outside their frames: sa_attn_item.text_window), 3D rotary
 * position embedding over (t, h, w) and 16 heads of 128 dimensions.
 *   Source: "Hy-Nomas: an 8.6B world model whose memory is a KV cache"
 *   (ai.thesatyajit.com), sections "How one segment is made" (token grid,
 *   heads, RoPE split [16, 56, 56] with theta 256, segment-wise causal joint
 *   attention reading history from a KV cache), "Writing the segment into
 *   memory" (a finished segment's K/V are written to the cache),
 *   "What 'world memory' stores" (per-layer K/V of past video and text
 *   tokens) and "The 4090 preset" (a power-spaced pick of past frames is
 *   restored before each segment; the cache is stored quantised and
 *   computed in BF16).
 *
 * Conventions shared by every call.
 *  - Device pointers are raw HIP device addresses owned by the caller; the
 *    library allocates no memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Device calls are asynchronous: buffers must stay alive until the stream
 *    has passed the call.
 *  - Every call validates its arguments on the host before any HIP call and
 *    returns an sa_status; on failure nothing is launched and
 *    sa_last_error() describes the problem (thread-local, valid until the
 *    next sa_* call on the same thread). Launch failures return SA_E_HIP.
 *  - Device-side index lists (frame lists, block lists) are trusted by this
 *    library: frame entries must lie in [0, frame_capacity) of the layer they
 *    index, block entries as sa_attn_item.block_list states;
 *    sa_history_select and sa_sparse_select only produce such lists. The
 *    debug build of the same ABI (libsegattn_debug.so, host code compiled
 *    with SA_DEBUG_CHECKS) copies each list to the host on the call's stream
 *    and waits for it before the launch that reads it, refuses a bad entry
 *    (SA_E_RANGE; SA_E_ARG for a block repeated in one list), and fills the
 *    attention outputs with NaN before the kernels write them. It is for
 *    finding bad lists, not for graph capture or speed.
 *  - bf16 = bfloat16 (raw 16-bit patterns); e4m3 = OCP 8-bit float e4m3fn
 *    (bias 7, max 448, no infinities).
 *  - Results are bitwise reproducible run to run (no atomics, fixed
 *    reduction orders).
 */
#ifndef SEGATTN_H
#define SEGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 11
#define SA_HEAD_DIM 128       /* the only head dim the kernels are built for */
#define SA_MAX_ITEMS 8        /* sessions per sa_segment_attention call     */
#define SA_MAX_FRAMES_KV 65536
#define SA_WINDOW_TABLE_WORDS 2048   /* bound on timed text windows, see below  */
#define SA_SPARSE_KEY_BLOCK 64       /* keys per candidate history block          */
#define SA_SPARSE_QUERY_BLOCK 256    /* query rows that share one block list      */
#define SA_MAX_SPARSE_CANDIDATES 8192 /* candidate blocks sa_sparse_select ranks  */
#define SA_MAX_CAMERA_CHUNK 16       /* latent frames per camera chunk            */

typedef enum {
  SA_OK = 0,
  SA_E_ARG = 1,          /* null pointer, negative count, bad enum        */
  SA_E_SHAPE = 2,        /* geometry not supported (head_dim, split, P)   */
  SA_E_ALIGN = 3,        /* pointer not 16-byte aligned                   */
  SA_E_UNSUPPORTED = 4,  /* dtype / feature combination not built         */
  SA_E_RANGE = 5,        /* frame index or count outside the layer        */
  SA_E_CAPACITY = 6,     /* output buffer too small                       */
  SA_E_HIP = 7           /* a HIP runtime call or launch failed           */
} sa_status;

typedef enum { SA_KV_BF16 = 0, SA_KV_FP8_E4M3 = 1, SA_KV_INT8 = 2 } sa_kv_dtype;

typedef enum {
  SA_SEL_ALL = 0,            /* every past frame                              */
  SA_SEL_RECENT = 1,         /* the newest `budget` frames                    */
  SA_SEL_POWER = 2,          /* power-spaced pick ("The 4090 preset")         */
  SA_SEL_ANCHOR_RECENT = 3   /* first frame of each segment + newest segments */
} sa_sel_policy;

/* Attention geometry, identical for every layer of a model.
 *   heads          number of heads H (16 in the pages' model)
 *   head_dim       must be SA_HEAD_DIM (128)
 *   lat_h, lat_w   latent frame grid; P = lat_h * lat_w tokens per frame
 *                  (22 x 40 = 880 in the pages' model). P % 8 == 0 is required.
 *   rope_split     dims of the t, h, w bands; each even, sum == head_dim
 *   rope_theta     RoPE base (> 1); band a, pair j rotates by
 *                  pos_a * theta^(-2j / rope_split[a]); pairs are (2j, 2j+1)
 *   softmax_scale  logit scale; 0 selects 1/sqrt(head_dim)                 */
typedef struct sa_geom {
  int32_t heads;
  int32_t head_dim;
  int32_t lat_h;
  int32_t lat_w;
  int32_t rope_split[3];
  float rope_theta;
  float softmax_scale;
} sa_geom;

/* One layer's cache planes (device memory, caller-allocated; sizes from
 * sa_cache_bytes / the shapes below). Frames are addressed by their absolute
 * latent-frame index since the world started, which is also their RoPE t.
 *   k        [frame_capacity][H][PL][128]        rotated keys
 *   v        [frame_capacity][H][128][PL]        values, transposed per
 *                                                (frame, head)
 *   k_text   [H][text_capacity][128]             text keys (no rotation)
 *   v_text   [H][128][text_capacity]             text values, transposed
 *   k_scale, v_scale            fp8: [frame_capacity][H] fp32 (one per
 *                               plane); int8: [frame_capacity][H][PL] fp32
 *                               (one per token and head)
 *   k_text_scale, v_text_scale  fp8: [H]; int8: [H][text_capacity]
 *                               (NULL for bf16)
 * PL, the token slots of a frame plane, is P for bf16 and P rounded up to a
 * multiple of 16 for e4m3 and int8 (so every V^T row starts 16-byte
 * aligned): slots p >= P hold zero V^T codes and zero int8 scales, written by
 * sa_kv_append; their K rows are never read. For P % 16 == 0, PL = P.
 * Element type: bf16 (2 bytes), e4m3 or int8 (1 byte) per `dtype`. int8 is
 * the pages' single-GPU cache format ("The 4090 preset": a byte per value
 * and an fp32 scale for each token and head, 4,224 bytes per token and layer
 * at 16 heads). text_capacity must be a multiple of 16; it may be 0 (no text
 * slot).                                                                    */
typedef struct sa_kv_layer {
  int32_t dtype;
  int32_t frame_capacity;
  int32_t text_capacity;
  int32_t reserved0;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  void* k_text;
  void* v_text;
  float* k_text_scale;
  float* v_text_scale;
} sa_kv_layer;

/* One session's attention call.
 *   q          bf16 [n_frames_q * P + n_text_q][H][128]: raw (unrotated)
 *              queries, video tokens in (t, h, w) raster order, then text
 *   frame0_q   absolute frame index (RoPE t) of the first query frame
 *   kv         that session's cache layer
 *   frames     device int32 [n_frames_kv]: the frames whose keys are
 *              attended, in order (kept history, then the current segment,
 *              which must already have been appended)
 *   n_text_kv  number of text keys taken from the layer's text slot
 *   out        bf16, same shape as q
 *   lse        optional fp32 [rows][H] natural-log sum of exp of the scaled
 *              logits per row and head (NULL to skip)
 *   text_window optional device int32 [n_text_kv][2]: timed text windows.
 *              Text key j is visible to a video query of absolute frame t
 *              only if text_window[2j] <= t <= text_window[2j + 1]; text
 *              queries see every text key. NULL: every query sees every key.
 *              ("How one segment is made", its second mask: the text of an
 *              action that has a time window is hidden from video frames
 *              outside that window.) 8-byte aligned; read
 *              on the stream by this call's kernels. With video queries and text keys the
 *              item needs n_frames_kv >= 1 (SA_E_ARG otherwise: a video
 *              query sees at least its own segment's frames), and
 *              (255 / P + 3) * ceil(n_text_kv / 32) <= SA_WINDOW_TABLE_WORDS
 *              (SA_E_RANGE otherwise; frames of 128 tokens allow 16384 text
 *              keys, frames of 16 tokens 3616).
 *   block_list optional device int32 [H][ceil(rows / 256)][keep_blocks]:
 *              block-sparse history ("Hy-Nomas en una RTX 4090", "El preset
 *              de una GPU": after the first denoising steps only a quarter of
 *              the candidate video blocks are attended). The candidates are
 *              the first n_hist_frames entries of `frames`, each cut into
 *              blocks of SA_SPARSE_KEY_BLOCK tokens (the last block of a frame
 *              is shorter when 64 does not divide P); block b of frame-list
 *              position f, in-frame index j, is f * ceil(P / 64) + j. Query
 *              rows [256 i, 256 i + 256) of head h attend only the candidate
 *              blocks listed at [h][i], plus every key after the history
 *              (the remaining frames and the text). Entries must be distinct
 *              and lie in [0, n_hist_frames * ceil(P / 64)); ascending order
 *              reads the cache in order. NULL: dense. sa_sparse_select
 *              writes such lists. 4-byte aligned.
 *   n_hist_frames, keep_blocks: the candidate frames and the list length
 *              (1 <= keep_blocks <= candidates); ignored when block_list is
 *              NULL or n_hist_frames is 0.
 * At least one key is required (n_frames_kv * P + n_text_kv >= 1).         */
typedef struct sa_attn_item {
  const void* q;
  int32_t frame0_q;
  int32_t n_frames_q;
  int32_t n_text_q;
  int32_t reserved0;
  const sa_kv_layer* kv;
  const int32_t* frames;
  int32_t n_frames_kv;
  int32_t n_text_kv;
  void* out;
  float* lse;
  const int32_t* text_window;
  const int32_t* block_list;
  int32_t n_hist_frames;
  int32_t keep_blocks;
} sa_attn_item;

int sa_abi_version(void);
const char* sa_last_error(void);
const char* sa_status_string(int status);

/* Bytes of one layer's cache planes in this layout (K + V planes, text slot,
 * and for fp8 / int8 the fp32 scales). For bf16 a token costs 2 * H * 128 * 2
 * bytes per layer, the 8,192 bytes of "What 'world memory' stores" at 16
 * heads; for int8, with a scale per token and head for K and V, the 4,224
 * bytes of "The 4090 preset". A frame counts PL token slots (see
 * sa_kv_layer). Returns 0 and sets the error on bad input
 * (SA_E_SHAPE geometry, SA_E_UNSUPPORTED dtype, SA_E_ARG negative capacity). */
size_t sa_cache_bytes(const sa_geom* geom, int32_t dtype, int32_t frame_capacity,
                      int32_t text_capacity);

/* kv_append: write frames [frame0, frame0 + n_frames) of one segment into the
 * layer. k_in, v_in: bf16 [n_frames * P][H][128], raw projections in raster
 * order. K is rotated by the 3D RoPE at (frame, row, column) in fp32 with an
 * fp64-reduced angle, then rounded to the cache type; V is stored unrotated
 * and transposed. fp8: per (frame, head) plane, scale = 2^e (an fp32 power
 * of two), e the least integer with amax <= 448 * 2^e and at least -126;
 * code = round-nearest-even(x * 2^-e), an exact product; amax 0 gives scale
 * 1. int8: per token and head, scale = amax / 127 over its 128 values, code
 * = round-half-even(x * (127 / amax)) clamped to +-127, in fp32 (K after its
 * rotation in fp32); amax 0 gives scale 1 and codes 0. Source: "Writing the segment into memory" and "How one segment is made"
 * (RoPE). Errors: SA_E_RANGE if frame0 < 0 or frame0 + n_frames >
 * frame_capacity.                                                           */
sa_status sa_kv_append(const sa_geom* geom, const sa_kv_layer* layer, const void* k_in,
                       const void* v_in, int32_t frame0, int32_t n_frames, void* stream);

/* text_append: write n_text text tokens into the layer's text slot (no
 * rotation: text sits at position (0,0,0)). k_in, v_in: bf16 [n_text][H][128].
 * Source: "How one segment is made" (the segment's text tokens join its
 * video tokens in the joint attention) and "What 'world memory' stores" (the
 * cache keeps text tokens' keys and values as well as video tokens').
 * fp8: one scale per head over the n_text tokens; int8: one per token and
 * head, and the tokens [n_text, capacity) get zero codes and zero scales.
 * Slots [n_text, capacity) of the value plane are zeroed so that a partial
 * last key chunk reads finite values. Errors: SA_E_CAPACITY if n_text >
 * text_capacity.                                                            */
sa_status sa_text_append(const sa_geom* geom, const sa_kv_layer* layer, const void* k_in,
                         const void* v_in, int32_t n_text, void* stream);

/* history_select (host only, pure): the kept past frames for a history of
 * t_past latent frames, sorted ascending, written to out_frames[0..*out_n).
 *   SA_SEL_ALL            every frame (budget, gamma ignored)
 *   SA_SEL_RECENT         the newest min(budget, t_past) frames
 *   SA_SEL_POWER          N = min(budget, t_past); kept = t_past-1-d_i with
 *                         d_i = i + rint((t_past-N) * (i/(N-1))^gamma)
 *                         ("The 4090 preset"); N == t_past keeps all, N == 1
 *                         keeps the newest
 *   SA_SEL_ANCHOR_RECENT  frame s*F of every F-frame segment plus all frames
 *                         of the newest `recent_segments` segments
 *                         (F = frames_per_segment)
 * Errors: SA_E_CAPACITY if the result does not fit in cap entries.         */
sa_status sa_history_select(int32_t policy, int32_t t_past, int32_t budget, double gamma,
                            int32_t frames_per_segment, int32_t recent_segments,
                            int32_t* out_frames, int32_t cap, int32_t* out_n);

/* history_gather: materialise frames[i] of src into frame slot i of dst
 * (i < n), K and V planes and, for fp8 / int8, their scales; a byte copy.
 * dst must have the same dtype and frame_capacity >= n. d_frames is a device
 * array of n entries in [0, src->frame_capacity) (trusted, as every frame
 * list). Source: "The 4090 preset" (before each segment only the picked past
 * frames are brought back from the archive to the GPU); this is that step for
 * callers that want a compact buffer, while sa_segment_attention reads the
 * picked frames in place through a frame list.
 * Errors: SA_E_UNSUPPORTED (dtypes differ), SA_E_CAPACITY (n > dst capacity),
 * SA_E_RANGE (src has no frames), SA_E_ARG.                                 */
sa_status sa_history_gather(const sa_geom* geom, const sa_kv_layer* src, const int32_t* d_frames,
                            int32_t n, const sa_kv_layer* dst, void* stream);

/* segment_attention: for every item, head and query row,
 *   out = softmax(scale * rope(q) . K^T) V over the item's key set
 * (frames list in order, then n_text_kv text keys), fp32 accumulation, bf16
 * output. bf16 layers use bf16 MFMA; fp8 layers use fp8 MFMA with queries
 * split per (row, head) into an e4m3 high part and an e4m3 low part (scaled
 * by 2^-4), and the per-(frame, head) scales applied to the logits and folded
 * into the probabilities. int8 layers run the bf16 path: each key tile is
 * dequantised (code * its token's scale, rounded to bf16) as it is staged,
 * so the cache stays narrow while the arithmetic is BF16 ("El preset de una
 * GPU"). All items must share one dtype.
 * Work is split into 256-row query tiles per (item, head). When the tiles do
 * not fill the device evenly, the tiles of the last partial round are split
 * further over their key range, and a second kernel merges the partial
 * results (max, sum and unnormalised output per row, combined in fixed order:
 * results are deterministic). The partials live in the caller's workspace of
 * sa_segment_attention_workspace() bytes (device memory, 16-byte aligned,
 * owned by the caller, overlapping no input or output; calls that share one
 * workspace must not overlap in time). With a smaller, unaligned or NULL
 * workspace nothing is split and the result is the same up to rounding.
 * sa_segment_attention_workspace returns 0 when no split pays, when the
 * arguments are invalid (sa_segment_attention then reports the error) or
 * when no device is current; it launches nothing.
 * Source: "How one segment is made" and "What 'world memory' stores".
 * Errors: SA_E_ARG (n_items outside [1, SA_MAX_ITEMS], empty key set),
 * SA_E_RANGE (n_frames_kv > SA_MAX_FRAMES_KV, n_text_kv > text_capacity).   */
size_t sa_segment_attention_workspace(const sa_geom* geom, const sa_attn_item* items,
                                      int32_t n_items);
sa_status sa_segment_attention(const sa_geom* geom, const sa_attn_item* items, int32_t n_items,
                               void* workspace, size_t workspace_bytes, void* stream);

/* segment_attention_counted: sa_segment_attention (the same joint attention
 * of "How one segment is made" over the cache of "What 'world memory'
 * stores"), plus diagnostic counts added (not stored: the caller clears
 * them) into counters, device uint32 [3], 4-byte aligned:
 *   [0] work tiles run (a query tile of one head, or one key-range part);
 *   [1] slow-path events: bf16 and int8 caches, work tiles whose key loop
 *       ran a second time with per-block rescaling (some row's block sum of
 *       probabilities, taken against the first block's max, passed 2^64);
 *       e4m3 cache, renormalisations of a wave's output (its running max
 *       rose more than 64 log2 units above the first tile's max);
 *   [2] rescale steps of waves: bf16 and int8, in that second run, blocks
 *       whose probability sum passed 256 and moved the running max; e4m3,
 *       blocks whose largest scaled probability passed 2^8.5 and moved it.
 * The outputs are those of sa_segment_attention bit for bit; the counts
 * tell how often softmax's rescaling paths ran (they are rare for
 * near-uniform attention and frequent for sharp logits). The extra cost is
 * one integer add per wave. Errors: those of sa_segment_attention; SA_E_ARG
 * (counters NULL), SA_E_ALIGN.                                              */
sa_status sa_segment_attention_counted(const sa_geom* geom, const sa_attn_item* items,
                                       int32_t n_items, void* workspace, size_t workspace_bytes,
                                       uint32_t* counters, void* stream);

/* sparse_select: block lists for block-sparse history attention. For every
 * head h and query block i (rows [256 i, 256 i + 256) of the item, video then
 * text), the score of candidate block b (see sa_attn_item.block_list) is
 *   mean over the block's rows of rope(q)  .  mean over the block's keys of K
 * (K as stored: rotated, and for e4m3 codes times the plane's scale), in
 * fp32; the keep_blocks best scores are kept (ties to the lower index) and
 * written in ascending order to block_list [H][ceil(rows / 256)][keep_blocks].
 * Uses item->q, kv, frames, frame0_q, n_frames_q, n_text_q, n_hist_frames
 * and keep_blocks (its block_list field is ignored). The pooled keys live in
 * the caller's workspace of sa_sparse_select_workspace() bytes (device, 16-byte
 * aligned). Source: "El preset de una GPU" (sparse attention keeps 25 % of the
 * candidate video blocks); the block size, the query block and the pooled
 * score are readings, not stated on the pages.
 * Errors: SA_E_ARG (no candidates, keep_blocks outside [1, candidates], no
 * query rows), SA_E_RANGE (candidates > SA_MAX_SPARSE_CANDIDATES,
 * n_hist_frames > n_frames_kv), SA_E_CAPACITY (workspace too small),
 * SA_E_ALIGN.                                                               */
size_t sa_sparse_select_workspace(const sa_geom* geom, const sa_attn_item* item);
sa_status sa_sparse_select(const sa_geom* geom, const sa_attn_item* item, void* workspace,
                           size_t workspace_bytes, int32_t* block_list, void* stream);

/* sparse_select_noalloc: sa_sparse_select for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels, the same block lists bit for bit,
 * but the pooled keys live in the library's own static device array of
 * SA_SPARSE_SCRATCH_BYTES bytes (one per GPU, held until the process ends)
 * instead of a caller workspace. The caller still passes the inputs and the
 * output block_list. No allocation of any kind happens in the call (the
 * array's device address is looked up once per device, on the first call
 * with that device current). The array needs no clearing: each call writes
 * every pooled key it reads. All calls on one GPU share the array, so calls
 * that overlap in time on one GPU (two streams, two threads) race; calls on
 * one stream are ordered. Errors: those of sa_sparse_select, except that
 * SA_E_CAPACITY means heads x candidate blocks x 512 bytes exceeds
 * SA_SPARSE_SCRATCH_BYTES (at most 65,536 head-candidate pairs: e.g. 16
 * heads x 4,096 candidates); SA_E_HIP if the array's address lookup fails.  */
#define SA_SPARSE_SCRATCH_BYTES (32u << 20)
sa_status sa_sparse_select_noalloc(const sa_geom* geom, const sa_attn_item* item,
                                   int32_t* block_list, void* stream);

/* sparse_keep: how many of n_candidates history blocks a block-sparse pass
 * keeps at `percent` (the pages keep 25 % of the candidate video blocks):
 * ceil(n_candidates * percent / 100), at least 1 and at most n_candidates;
 * 0 for n_candidates <= 0. percent must lie in [1, 100] (else -1 and the
 * error is set). Host only, pure.                                           */
int32_t sa_sparse_keep(int32_t n_candidates, int32_t percent);

/* camera_attention: cross-attention of the segment's video tokens to the
 * camera tokens, one per latent frame ("Hy-Nomas: an 8.6B world model ...",
 * section "The camera": a small cross-attention after each block; with chunk
 * size 1 the mask is block-diagonal, latent frame t attends only to its own
 * camera token; the camera key/value projection is 2,048 x 128).
 *   q        bf16 [n_frames * P][H][128] video queries, (t, h, w) raster order
 *            (no rotary embedding)
 *   cam_k, cam_v  bf16 [n_cam][kv_heads][128]; kv_heads = 1 (one head shared
 *            by every query head) or H; token i belongs to latent frame i
 *   out      bf16 like q;  lse  optional fp32 [n_frames * P][H] (NULL: skip)
 * Rows of latent frame t attend to camera tokens c * floor(t / c) ..
 * min(n_cam, c * floor(t / c) + c) - 1, c = chunk, softmax scale from geom.
 * Pointers 16-byte aligned. Errors: SA_E_ARG (n_frames < 1, chunk outside
 * [1, SA_MAX_CAMERA_CHUNK], n_cam < n_frames, kv_heads not 1 or H, NULL
 * pointers), SA_E_ALIGN.                                                    */
sa_status sa_camera_attention(const sa_geom* geom, const void* q, int32_t n_frames,
                              const void* cam_k, const void* cam_v, int32_t n_cam,
                              int32_t kv_heads, int32_t chunk, void* out, float* lse,
                              void* stream);

/* kv_dequant: fp8 frames[i] of src -> bf16 frame slot i of dst (K and V
 * planes: value = code * scale, rounded to bf16), and, when n_text > 0, the
 * first n_text tokens of the text slot; the destination's text value plane
 * gets zeros in its columns [n_text, dst->text_capacity), so that attention
 * over the first n_text text keys reads finite values there (the K rows
 * past n_text are never read). The pages' route of a cache kept in a narrow
 * format with BF16 arithmetic ("El preset de una GPU", inferencekey.com).
 * src may also be int8 (value = code * the token's scale).
 * dst must be a bf16 layer with frame_capacity >= n_frames and
 * text_capacity >= n_text. Errors: SA_E_UNSUPPORTED (src bf16 or dst not
 * bf16), SA_E_CAPACITY, SA_E_RANGE (src has no frames), SA_E_ARG.          */
sa_status sa_kv_dequant(const sa_geom* geom, const sa_kv_layer* src, const int32_t* d_frames,
                        int32_t n_frames, int32_t n_text, const sa_kv_layer* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SEGATTN_H */
