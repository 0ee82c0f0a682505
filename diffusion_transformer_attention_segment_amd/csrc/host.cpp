// Host side of the C ABI: argument validation, launch configuration and the
// host-only history selection. Every entry point validates before any HIP
// call and reports failures through a status code plus a thread-local message.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <set>
#include <string>
#include <vector>

#include "internal.h"

using namespace segattn;

namespace {

thread_local std::string g_err;

sa_status fail(sa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sa_status ok() {
  g_err.clear();
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sa_status check_geom(const sa_geom* g) {
  if (g == nullptr) return fail(SA_E_ARG, "geom is NULL");
  if (g->head_dim != SA_HEAD_DIM)
    return fail(SA_E_SHAPE, "head_dim %d unsupported (only %d)", g->head_dim, SA_HEAD_DIM);
  if (g->heads < 1 || g->heads > 1024) return fail(SA_E_SHAPE, "heads %d out of range", g->heads);
  if (g->lat_h < 1 || g->lat_w < 1) return fail(SA_E_SHAPE, "latent grid %dx%d", g->lat_h, g->lat_w);
  const int64_t P = static_cast<int64_t>(g->lat_h) * g->lat_w;
  if (P % 8 != 0 || P > (1 << 20))
    return fail(SA_E_SHAPE, "tokens per frame P=%lld must be a multiple of 8 (and <= 2^20)",
                static_cast<long long>(P));
  int sum = 0;
  for (int i = 0; i < 3; ++i) {
    if (g->rope_split[i] < 0 || g->rope_split[i] % 2 != 0)
      return fail(SA_E_SHAPE, "rope_split[%d]=%d must be even and >= 0", i, g->rope_split[i]);
    sum += g->rope_split[i];
  }
  if (sum != g->head_dim) return fail(SA_E_SHAPE, "rope_split sums to %d, not head_dim", sum);
  if (!(g->rope_theta > 1.0f) || !std::isfinite(g->rope_theta))
    return fail(SA_E_SHAPE, "rope_theta must be finite and > 1");
  if (!(g->softmax_scale >= 0.0f) || !std::isfinite(g->softmax_scale))
    return fail(SA_E_SHAPE, "softmax_scale must be finite and >= 0");
  return SA_OK;
}

int32_t tokens_per_frame(const sa_geom* g) { return g->lat_h * g->lat_w; }

// Token slots of one (frame, head) plane of a layer of this dtype.
int32_t frame_slots(const sa_geom* g, int32_t dtype) {
  return plane_tokens(tokens_per_frame(g), dtype != SA_KV_BF16);
}

sa_status check_layer(const sa_geom* g, const sa_kv_layer* L, const char* name) {
  if (L == nullptr) return fail(SA_E_ARG, "%s layer is NULL", name);
  if (L->dtype != SA_KV_BF16 && L->dtype != SA_KV_FP8_E4M3 && L->dtype != SA_KV_INT8)
    return fail(SA_E_UNSUPPORTED, "%s: unknown dtype %d", name, L->dtype);
  const bool scaled = L->dtype != SA_KV_BF16;
  if (L->frame_capacity < 0 || L->text_capacity < 0)
    return fail(SA_E_ARG, "%s: negative capacity", name);
  if (L->text_capacity % 16 != 0)
    return fail(SA_E_SHAPE, "%s: text_capacity %d must be a multiple of 16", name, L->text_capacity);
  if (L->frame_capacity > 0) {
    if (L->k == nullptr || L->v == nullptr) return fail(SA_E_ARG, "%s: k/v plane is NULL", name);
    if (!aligned16(L->k) || !aligned16(L->v)) return fail(SA_E_ALIGN, "%s: k/v not 16-byte aligned", name);
    if (scaled && (L->k_scale == nullptr || L->v_scale == nullptr))
      return fail(SA_E_ARG, "%s: fp8 and int8 layers need k_scale and v_scale", name);
  }
  if (L->text_capacity > 0) {
    if (L->k_text == nullptr || L->v_text == nullptr)
      return fail(SA_E_ARG, "%s: text slot pointers are NULL", name);
    if (!aligned16(L->k_text) || !aligned16(L->v_text))
      return fail(SA_E_ALIGN, "%s: text slot not 16-byte aligned", name);
    if (scaled && (L->k_text_scale == nullptr || L->v_text_scale == nullptr))
      return fail(SA_E_ARG, "%s: fp8 and int8 text slots need scales", name);
  }
  return SA_OK;
}

RopeParams rope_params(const sa_geom* g) {
  RopeParams r;
  r.split0 = g->rope_split[0];
  r.split1 = g->rope_split[1];
  r.split2 = g->rope_split[2];
  r.lat_w = g->lat_w;
  r.P = tokens_per_frame(g);
  r.log2_theta = std::log2(static_cast<double>(g->rope_theta));
  return r;
}

hipError_t launch_append(int32_t dtype, const AppendArgs& a, hipStream_t s) {
  if (dtype == SA_KV_BF16) return launch_append_bf16(a, s);
  if (dtype == SA_KV_INT8) return launch_append_int8(a, s);
  return launch_append_fp8(a, s);
}

sa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#ifdef SA_DEBUG_CHECKS
// Debug builds check what release builds trust: the device index lists are
// copied to the host on the call's stream (the call then waits for that
// stream) and every entry must lie in [0, hi); with distinct_rows, each run
// of `row` entries must hold distinct values.
sa_status debug_check_list(const int32_t* d, int64_t n, int64_t row, int32_t hi, bool distinct_rows,
                           hipStream_t s, const char* what) {
  if (n <= 0) return SA_OK;
  std::vector<int32_t> h(static_cast<size_t>(n));
  hipError_t e = hipMemcpyAsync(h.data(), d, static_cast<size_t>(n) * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, what);
  for (int64_t i = 0; i < n; ++i)
    if (h[i] < 0 || h[i] >= hi)
      return fail(SA_E_RANGE, "%s: entry %lld is %d, outside [0, %d) (debug check)", what,
                  static_cast<long long>(i), h[i], hi);
  if (distinct_rows) {
    for (int64_t r0 = 0; r0 < n; r0 += row) {
      std::vector<int32_t> v(h.begin() + r0, h.begin() + std::min(n, r0 + row));
      std::sort(v.begin(), v.end());
      if (std::adjacent_find(v.begin(), v.end()) != v.end())
        return fail(SA_E_ARG, "%s: row %lld repeats an entry (debug check)", what,
                    static_cast<long long>(r0 / row));
    }
  }
  return SA_OK;
}

// Frame lists and block lists of an attention call, then NaN canaries in
// every output row (bf16 and fp32 all-ones bytes are NaN), so that a row the
// kernels leave unwritten shows in the result.
sa_status debug_check_attention(const sa_geom* geom, const sa_attn_item* items, int32_t n_items,
                                hipStream_t s) {
  const int32_t P = tokens_per_frame(geom);
  char what[64];
  for (int i = 0; i < n_items; ++i) {
    const sa_attn_item& it = items[i];
    std::snprintf(what, sizeof what, "item %d frames", i);
    sa_status st = debug_check_list(it.frames, it.n_frames_kv, 1, it.kv->frame_capacity, false, s,
                                    what);
    if (st != SA_OK) return st;
    const int64_t rows = static_cast<int64_t>(it.n_frames_q) * P + it.n_text_q;
    if (it.block_list != nullptr && it.n_hist_frames > 0) {
      const int64_t qb = (rows + SA_SPARSE_QUERY_BLOCK - 1) / SA_SPARSE_QUERY_BLOCK;
      const int32_t cand = it.n_hist_frames * ((P + 63) / 64);
      std::snprintf(what, sizeof what, "item %d block_list", i);
      st = debug_check_list(it.block_list, geom->heads * qb * it.keep_blocks, it.keep_blocks, cand,
                            true, s, what);
      if (st != SA_OK) return st;
    }
    if (rows > 0) {
      const size_t vals = static_cast<size_t>(rows) * geom->heads;
      hipError_t e = hipMemsetAsync(it.out, 0xFF, vals * geom->head_dim * sizeof(uint16_t), s);
      if (e == hipSuccess && it.lse != nullptr) e = hipMemsetAsync(it.lse, 0xFF, vals * sizeof(float), s);
      if (e != hipSuccess) return hip_status(e, "attention output canary");
    }
  }
  return SA_OK;
}
#endif

}  // namespace

extern "C" {

int sa_abi_version(void) { return SA_ABI_VERSION; }

const char* sa_last_error(void) { return g_err.c_str(); }

const char* sa_status_string(int status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_E_ARG: return "SA_E_ARG";
    case SA_E_SHAPE: return "SA_E_SHAPE";
    case SA_E_ALIGN: return "SA_E_ALIGN";
    case SA_E_UNSUPPORTED: return "SA_E_UNSUPPORTED";
    case SA_E_RANGE: return "SA_E_RANGE";
    case SA_E_CAPACITY: return "SA_E_CAPACITY";
    case SA_E_HIP: return "SA_E_HIP";
    default: return "unknown status";
  }
}

size_t sa_cache_bytes(const sa_geom* geom, int32_t dtype, int32_t frame_capacity,
                      int32_t text_capacity) {
  if (check_geom(geom) != SA_OK) return 0;
  if (dtype != SA_KV_BF16 && dtype != SA_KV_FP8_E4M3 && dtype != SA_KV_INT8) {
    fail(SA_E_UNSUPPORTED, "unknown dtype %d", dtype);
    return 0;
  }
  if (frame_capacity < 0 || text_capacity < 0) {
    fail(SA_E_ARG, "negative capacity");
    return 0;
  }
  const size_t H = geom->heads, D = geom->head_dim, P = frame_slots(geom, dtype);
  const size_t elems = 2 * H * D * (static_cast<size_t>(frame_capacity) * P + text_capacity);
  ok();
  if (dtype == SA_KV_BF16) return 2 * elems;
  if (dtype == SA_KV_INT8)   // a scale per token and head, K and V
    return elems + 2 * sizeof(float) * H * (static_cast<size_t>(frame_capacity) * P + text_capacity);
  return elems + 2 * sizeof(float) * H * (static_cast<size_t>(frame_capacity) + 1);
}

sa_status sa_kv_append(const sa_geom* geom, const sa_kv_layer* layer, const void* k_in,
                       const void* v_in, int32_t frame0, int32_t n_frames, void* stream) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if ((st = check_layer(geom, layer, "kv_append")) != SA_OK) return st;
  if (n_frames < 0) return fail(SA_E_ARG, "n_frames %d < 0", n_frames);
  if (frame0 < 0 || static_cast<int64_t>(frame0) + n_frames > layer->frame_capacity)
    return fail(SA_E_RANGE, "frames [%d, %lld) outside capacity %d", frame0,
                static_cast<long long>(frame0) + n_frames, layer->frame_capacity);
  if (n_frames == 0) return ok();
  if (k_in == nullptr || v_in == nullptr) return fail(SA_E_ARG, "k_in/v_in is NULL");
  if (!aligned16(k_in) || !aligned16(v_in)) return fail(SA_E_ALIGN, "k_in/v_in not 16-byte aligned");
  AppendArgs a{};
  a.k_in = static_cast<const uint16_t*>(k_in);
  a.v_in = static_cast<const uint16_t*>(v_in);
  a.k = layer->k;
  a.v = layer->v;
  a.k_scale = layer->k_scale;
  a.v_scale = layer->v_scale;
  a.heads = geom->heads;
  a.frame0 = frame0;
  a.n_frames = n_frames;
  a.plane_len = frame_slots(geom, layer->dtype);
  a.n_tok = tokens_per_frame(geom);
  a.is_text = 0;
  a.rope = rope_params(geom);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_append(layer->dtype, a, s), "kv_append launch");
}

sa_status sa_text_append(const sa_geom* geom, const sa_kv_layer* layer, const void* k_in,
                         const void* v_in, int32_t n_text, void* stream) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if ((st = check_layer(geom, layer, "text_append")) != SA_OK) return st;
  if (n_text < 0) return fail(SA_E_ARG, "n_text %d < 0", n_text);
  if (n_text > layer->text_capacity)
    return fail(SA_E_CAPACITY, "n_text %d > text_capacity %d", n_text, layer->text_capacity);
  if (layer->text_capacity == 0) return ok();
  if (n_text > 0 && (k_in == nullptr || v_in == nullptr)) return fail(SA_E_ARG, "k_in/v_in is NULL");
  if (n_text > 0 && (!aligned16(k_in) || !aligned16(v_in)))
    return fail(SA_E_ALIGN, "k_in/v_in not 16-byte aligned");
  AppendArgs a{};
  a.k_in = static_cast<const uint16_t*>(k_in);
  a.v_in = static_cast<const uint16_t*>(v_in);
  a.k = layer->k_text;
  a.v = layer->v_text;
  a.k_scale = layer->k_text_scale;
  a.v_scale = layer->v_text_scale;
  a.heads = geom->heads;
  a.frame0 = 0;
  a.n_frames = 1;
  a.plane_len = layer->text_capacity;
  a.n_tok = n_text;
  a.is_text = 1;
  a.rope = rope_params(geom);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(launch_append(layer->dtype, a, s), "text_append launch");
}

sa_status sa_history_select(int32_t policy, int32_t t_past, int32_t budget, double gamma,
                            int32_t frames_per_segment, int32_t recent_segments,
                            int32_t* out_frames, int32_t cap, int32_t* out_n) {
  if (out_n == nullptr) return fail(SA_E_ARG, "out_n is NULL");
  *out_n = 0;
  if (t_past < 0) return fail(SA_E_ARG, "t_past %d < 0", t_past);
  if (cap < 0 || (cap > 0 && out_frames == nullptr)) return fail(SA_E_ARG, "bad output buffer");
  std::vector<int32_t> sel;
  switch (policy) {
    case SA_SEL_ALL:
      for (int32_t f = 0; f < t_past; ++f) sel.push_back(f);
      break;
    case SA_SEL_RECENT: {
      if (budget < 0) return fail(SA_E_ARG, "budget %d < 0", budget);
      const int32_t n = budget < t_past ? budget : t_past;
      for (int32_t f = t_past - n; f < t_past; ++f) sel.push_back(f);
      break;
    }
    case SA_SEL_POWER: {
      if (budget < 0) return fail(SA_E_ARG, "budget %d < 0", budget);
      if (!(gamma > 0.0) || !std::isfinite(gamma)) return fail(SA_E_ARG, "gamma must be > 0");
      const int32_t N = budget < t_past ? budget : t_past;
      if (N == t_past) {
        for (int32_t f = 0; f < t_past; ++f) sel.push_back(f);
      } else if (N == 1) {
        sel.push_back(t_past - 1);
      } else if (N > 1) {
        // d_i = i + rint((T - N) * u_i^gamma), u_i = i / (N - 1); kept = T - 1 - d_i
        for (int32_t i = 0; i < N; ++i) {
          const double u = static_cast<double>(i) / static_cast<double>(N - 1);
          const double d = static_cast<double>(i) +
                           std::rint(static_cast<double>(t_past - N) * std::pow(u, gamma));
          sel.push_back(t_past - 1 - static_cast<int32_t>(d));
        }
        std::vector<int32_t> sorted(sel.rbegin(), sel.rend());
        sel.swap(sorted);
      }
      break;
    }
    case SA_SEL_ANCHOR_RECENT: {
      if (frames_per_segment < 1) return fail(SA_E_ARG, "frames_per_segment must be >= 1");
      if (recent_segments < 0) return fail(SA_E_ARG, "recent_segments < 0");
      const int64_t F = frames_per_segment;
      const int64_t n_seg = (t_past + F - 1) / F;
      const int64_t first_recent = n_seg - recent_segments > 0 ? n_seg - recent_segments : 0;
      for (int64_t f = 0; f < t_past; ++f)
        if (f % F == 0 || f / F >= first_recent) sel.push_back(static_cast<int32_t>(f));
      break;
    }
    default:
      return fail(SA_E_ARG, "unknown policy %d", policy);
  }
  if (static_cast<int64_t>(sel.size()) > cap)
    return fail(SA_E_CAPACITY, "selection has %zu frames, buffer holds %d", sel.size(), cap);
  if (!sel.empty()) std::memcpy(out_frames, sel.data(), sel.size() * sizeof(int32_t));
  *out_n = static_cast<int32_t>(sel.size());
  return ok();
}

sa_status sa_history_gather(const sa_geom* geom, const sa_kv_layer* src, const int32_t* d_frames,
                            int32_t n, const sa_kv_layer* dst, void* stream) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if ((st = check_layer(geom, src, "gather src")) != SA_OK) return st;
  if ((st = check_layer(geom, dst, "gather dst")) != SA_OK) return st;
  if (src->dtype != dst->dtype) return fail(SA_E_UNSUPPORTED, "gather: src and dst dtypes differ");
  if (n < 0) return fail(SA_E_ARG, "n %d < 0", n);
  if (n > dst->frame_capacity)
    return fail(SA_E_CAPACITY, "gather: %d frames > dst capacity %d", n, dst->frame_capacity);
  if (n == 0) return ok();
  if (d_frames == nullptr) return fail(SA_E_ARG, "frames is NULL");
  if (src->frame_capacity == 0) return fail(SA_E_RANGE, "gather: src has no frames");
  GatherArgs a{};
  a.src_k = src->k;
  a.src_v = src->v;
  a.dst_k = dst->k;
  a.dst_v = dst->v;
  const int64_t elt = src->dtype == SA_KV_BF16 ? 2 : 1;
  a.plane_bytes = elt * geom->heads * static_cast<int64_t>(frame_slots(geom, src->dtype)) * geom->head_dim;
  if (src->dtype != SA_KV_BF16) {
    a.src_ks = src->k_scale;
    a.src_vs = src->v_scale;
    a.dst_ks = dst->k_scale;
    a.dst_vs = dst->v_scale;
    a.scale_floats = src->dtype == SA_KV_INT8
                         ? static_cast<int64_t>(geom->heads) * frame_slots(geom, src->dtype)
                         : geom->heads;
  }
  a.frames = d_frames;
  a.n = n;
  a.heads = geom->heads;
  if (geom->heads > 256) return fail(SA_E_SHAPE, "gather: more than 256 heads");
#ifdef SA_DEBUG_CHECKS
  if ((st = debug_check_list(d_frames, n, 1, src->frame_capacity, false,
                             static_cast<hipStream_t>(stream), "gather frames")) != SA_OK)
    return st;
#endif
  return hip_status(launch_gather(a, static_cast<hipStream_t>(stream)), "history_gather launch");
}

namespace {

// Validated attention call: device arguments plus the per-item key-tile
// counts the split planner needs.
struct AttnPlan {
  AttnArgs a;
  bool fp8;
  int bm;
  int32_t key_tiles[SA_MAX_ITEMS];
};

// Timed text windows take effect only where a video query meets a text key.
bool windowed(const sa_attn_item& it) {
  return it.text_window != nullptr && it.n_text_kv > 0 && it.n_frames_q > 0;
}

// Block-sparse history takes effect when there are candidate frames.
bool sparse(const sa_attn_item& it) { return it.block_list != nullptr && it.n_hist_frames > 0; }

// Device view of a validated item (q_tiles and tile_begin are the caller's).
void fill_item(const sa_attn_item& it, int32_t P, AttnItemDev& d) {
  d = AttnItemDev{};
  d.q = static_cast<const uint16_t*>(it.q);
  d.out = static_cast<uint16_t*>(it.out);
  d.lse = it.lse;
  d.k = it.kv->k;
  d.v = it.kv->v;
  d.k_text = it.kv->k_text;
  d.v_text = it.kv->v_text;
  d.k_scale = it.kv->k_scale;
  d.v_scale = it.kv->v_scale;
  d.k_text_scale = it.kv->k_text_scale;
  d.v_text_scale = it.kv->v_text_scale;
  d.frames = it.frames;
  d.frame0_q = it.frame0_q;
  d.n_q_video = it.n_frames_q * P;
  d.n_q = d.n_q_video + it.n_text_q;
  d.n_frames_kv = it.n_frames_kv;
  d.n_text_kv = it.n_text_kv;
  d.text_cap = it.kv->text_capacity;
  d.text_window = windowed(it) ? it.text_window : nullptr;
  d.block_list = sparse(it) ? it.block_list : nullptr;
  d.n_hist_frames = sparse(it) ? it.n_hist_frames : 0;
  d.keep = sparse(it) ? it.keep_blocks : 0;
}

sa_status prepare_attention(const sa_geom* geom, const sa_attn_item* items, int32_t n_items,
                            AttnPlan& plan) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if (items == nullptr) return fail(SA_E_ARG, "items is NULL");
  if (n_items < 1 || n_items > SA_MAX_ITEMS)
    return fail(SA_E_ARG, "n_items %d outside [1, %d]", n_items, SA_MAX_ITEMS);
  const int32_t P = tokens_per_frame(geom);
  int32_t dtype = -1;
  for (int i = 0; i < n_items; ++i) {
    const sa_attn_item& it = items[i];
    if ((st = check_layer(geom, it.kv, "attention kv")) != SA_OK) return st;
    if (dtype == -1) dtype = it.kv->dtype;
    if (it.kv->dtype != dtype) return fail(SA_E_UNSUPPORTED, "items mix cache dtypes");
    if (it.n_frames_q < 0 || it.n_text_q < 0) return fail(SA_E_ARG, "item %d: negative query counts", i);
    if (it.frame0_q < 0) return fail(SA_E_ARG, "item %d: frame0_q < 0", i);
    if (it.n_frames_kv < 0 || it.n_text_kv < 0) return fail(SA_E_ARG, "item %d: negative key counts", i);
    if (it.n_frames_kv > SA_MAX_FRAMES_KV)
      return fail(SA_E_RANGE, "item %d: n_frames_kv %d > %d", i, it.n_frames_kv, SA_MAX_FRAMES_KV);
    if (it.n_frames_kv > 0 && it.kv->frame_capacity == 0)
      return fail(SA_E_RANGE, "item %d: frames given but the layer has no frame planes", i);
    if (it.n_text_kv > it.kv->text_capacity)
      return fail(SA_E_RANGE, "item %d: n_text_kv %d > text_capacity %d", i, it.n_text_kv,
                  it.kv->text_capacity);
    const int64_t lk = static_cast<int64_t>(it.n_frames_kv) * P + it.n_text_kv;
    if (lk < 1) return fail(SA_E_ARG, "item %d: empty key set", i);
    if (it.n_frames_kv > 0 && it.frames == nullptr) return fail(SA_E_ARG, "item %d: frames is NULL", i);
    if (windowed(it)) {
      if ((reinterpret_cast<uintptr_t>(it.text_window) & 7) != 0)
        return fail(SA_E_ALIGN, "item %d: text_window not 8-byte aligned", i);
      if (it.n_frames_kv == 0)
        return fail(SA_E_ARG, "item %d: timed text windows with video queries need video keys", i);
      const int wbm = dtype == SA_KV_FP8_E4M3 ? attention_block_m_fp8() : attention_block_m_bf16();
      const int words = window_table_rows(P, wbm) * window_row_words(it.n_text_kv);
      if (words > kWindowWords)
        return fail(SA_E_RANGE, "item %d: timed windows of %d text keys over frames of %d tokens "
                    "need %d table words > %d", i, it.n_text_kv, P, words, kWindowWords);
    }
    if (sparse(it)) {
      if (it.n_hist_frames > it.n_frames_kv)
        return fail(SA_E_RANGE, "item %d: n_hist_frames %d > n_frames_kv %d", i, it.n_hist_frames,
                    it.n_frames_kv);
      const int64_t cand = static_cast<int64_t>(it.n_hist_frames) * ((P + 63) / 64);
      if (it.keep_blocks < 1 || it.keep_blocks > cand)
        return fail(SA_E_ARG, "item %d: keep_blocks %d outside [1, %lld]", i, it.keep_blocks,
                    static_cast<long long>(cand));
      if ((reinterpret_cast<uintptr_t>(it.block_list) & 3) != 0)
        return fail(SA_E_ALIGN, "item %d: block_list not 4-byte aligned", i);
    }
    const int64_t rows = static_cast<int64_t>(it.n_frames_q) * P + it.n_text_q;
    if (rows > (int64_t(1) << 30)) return fail(SA_E_SHAPE, "item %d: too many query rows", i);
    if (rows > 0) {
      if (it.q == nullptr || it.out == nullptr) return fail(SA_E_ARG, "item %d: q/out is NULL", i);
      if (!aligned16(it.q) || !aligned16(it.out)) return fail(SA_E_ALIGN, "item %d: q/out not aligned", i);
    }
  }
  AttnArgs& a = plan.a;
  a = AttnArgs{};
  plan.fp8 = dtype == SA_KV_FP8_E4M3;
  a.int8 = dtype == SA_KV_INT8;   // bf16 kernel, tiles dequantised while staged
  plan.bm = plan.fp8 ? attention_block_m_fp8() : attention_block_m_bf16();
  const int bm = plan.bm;
  const int tpf = (P + 63) / 64;
  int64_t tiles = 0;
  for (int i = 0; i < n_items; ++i) {
    const sa_attn_item& it = items[i];
    AttnItemDev& d = a.items[i];
    fill_item(it, P, d);
    if (d.block_list != nullptr) a.any_sparse = 1;
    d.q_tiles = (d.n_q + bm - 1) / bm;
    d.tile_begin = static_cast<int32_t>(tiles);
    tiles += static_cast<int64_t>(d.q_tiles) * geom->heads;
    // key tiles a work tile visits (kept history blocks, then the rest); split
    // parts of an item with windows divide its video tiles only
    const int vid = sparse(it) ? d.keep + (it.n_frames_kv - it.n_hist_frames) * tpf
                               : it.n_frames_kv * tpf;
    plan.key_tiles[i] = vid + (windowed(it) ? 0 : (it.n_text_kv + 63) / 64);
  }
  if (tiles > (int64_t(1) << 31) - 1) return fail(SA_E_SHAPE, "too many tiles");
  a.n_items = n_items;
  a.heads = geom->heads;
  a.total_tiles = static_cast<int32_t>(tiles);
  a.n_full = a.total_tiles;
  a.split_k = 1;
  a.grid = a.total_tiles;
  const double scale = geom->softmax_scale > 0.f ? geom->softmax_scale : 1.0 / std::sqrt(128.0);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  a.rope = rope_params(geom);
  // items with no query rows own no tiles; point them past the end
  for (int i = n_items; i < SA_MAX_ITEMS; ++i) a.items[i].tile_begin = a.total_tiles;
  return ok();
}

// Compute units of the current device (cached per device; threads that race
// on the first query store the same value).
int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Split plan: the tiles of the last partial round (r = total mod CUs, or all
// tiles when there are fewer than CUs) are cut into k key-range parts, k in
// [2, 32] with at least 8 key tiles per part. k minimises the predicted time
// of that round in whole-tile units: rounds(r k) * (1/k + c0) + r k c1, where
// c0 ~ 3 key tiles of prologue per part and c1 ~ the merge's read of one
// part's fp32 partial (133 KB at ~5 TB/s against ~1.9 us per key tile), both
// relative to the tile's kt key tiles. Returns the workspace bytes (0: no
// split).
size_t plan_split(AttnPlan& plan) {
  AttnArgs& a = plan.a;
  const int cus = device_cus();
  const int T = a.total_tiles;
  if (cus <= 0 || T == 0) return 0;
  const int r = T >= cus ? T % cus : T;
  if (r == 0) return 0;
  const int first = T - r;
  int min_kt = 1 << 30;
  for (int i = 0; i < a.n_items; ++i) {
    const AttnItemDev& d = a.items[i];
    const int end = d.tile_begin + d.q_tiles * a.heads;
    if (end > first && d.q_tiles > 0) min_kt = std::min(min_kt, plan.key_tiles[i]);
  }
  const int kmax = std::min(32, min_kt / 8);
  const double c0 = 3.0 / min_kt, c1 = 0.014 / min_kt;
  double best = std::ceil(static_cast<double>(r) / cus);
  int best_k = 1;
  for (int k = 2; k <= kmax; ++k) {
    const double cost = std::ceil(static_cast<double>(r) * k / cus) * (1.0 / k + c0) +
                        static_cast<double>(r) * k * c1;
    if (cost < best - 1e-9) {
      best = cost;
      best_k = k;
    }
  }
  if (best_k == 1) return 0;
  a.n_full = first;
  a.split_k = best_k;
  a.grid = first + r * best_k;
  return static_cast<size_t>(r) * best_k * plan.bm * kPartialStride * sizeof(float);
}

}  // namespace

size_t sa_segment_attention_workspace(const sa_geom* geom, const sa_attn_item* items,
                                      int32_t n_items) {
  static thread_local AttnPlan plan;
  if (prepare_attention(geom, items, n_items, plan) != SA_OK) return 0;
  const size_t bytes = plan_split(plan);
  ok();
  return bytes;
}

namespace {

sa_status run_attention(const sa_geom* geom, const sa_attn_item* items, int32_t n_items,
                        void* workspace, size_t workspace_bytes, uint32_t* counters, void* stream) {
  static thread_local AttnPlan plan;
  sa_status st = prepare_attention(geom, items, n_items, plan);
  if (st != SA_OK) return st;
  AttnArgs& a = plan.a;
  a.counters = counters;
#ifdef SA_DEBUG_CHECKS
  if ((st = debug_check_attention(geom, items, n_items, static_cast<hipStream_t>(stream))) != SA_OK)
    return st;
#endif
  if (a.total_tiles == 0) return ok();
  const size_t need = plan_split(plan);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))) {
    a.n_full = a.total_tiles;   // no room for partials: run unsplit
    a.split_k = 1;
    a.grid = a.total_tiles;
  }
  a.ws = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(plan.fp8 ? launch_attention_fp8(a, s) : launch_attention_bf16(a, s),
                       "segment_attention launch")) != SA_OK)
    return st;
  if (a.split_k > 1)
    return hip_status(launch_attention_combine(a, plan.bm, s), "segment_attention combine launch");
  return ok();
}

}  // namespace

sa_status sa_segment_attention(const sa_geom* geom, const sa_attn_item* items, int32_t n_items,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return run_attention(geom, items, n_items, workspace, workspace_bytes, nullptr, stream);
}

sa_status sa_segment_attention_counted(const sa_geom* geom, const sa_attn_item* items,
                                       int32_t n_items, void* workspace, size_t workspace_bytes,
                                       uint32_t* counters, void* stream) {
  if (counters == nullptr) return fail(SA_E_ARG, "segment_attention_counted: counters is NULL");
  if ((reinterpret_cast<uintptr_t>(counters) & 3) != 0)
    return fail(SA_E_ALIGN, "segment_attention_counted: counters not 4-byte aligned");
  return run_attention(geom, items, n_items, workspace, workspace_bytes, counters, stream);
}

namespace {

// Validated block selection: kernel arguments and the pooled-key workspace size.
sa_status prepare_select(const sa_geom* geom, const sa_attn_item* item, SelectArgs& a,
                         size_t* ws_bytes) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if (item == nullptr) return fail(SA_E_ARG, "sparse_select: item is NULL");
  const sa_attn_item& it = *item;
  if ((st = check_layer(geom, it.kv, "sparse_select kv")) != SA_OK) return st;
  const int32_t P = tokens_per_frame(geom);
  if (it.n_frames_q < 0 || it.n_text_q < 0 || it.frame0_q < 0)
    return fail(SA_E_ARG, "sparse_select: negative query counts or frame0_q");
  const int64_t rows = static_cast<int64_t>(it.n_frames_q) * P + it.n_text_q;
  if (rows < 1) return fail(SA_E_ARG, "sparse_select: no query rows");
  if (rows > (int64_t(1) << 30)) return fail(SA_E_SHAPE, "sparse_select: too many query rows");
  if (it.q == nullptr) return fail(SA_E_ARG, "sparse_select: q is NULL");
  if (!aligned16(it.q)) return fail(SA_E_ALIGN, "sparse_select: q not 16-byte aligned");
  if (it.n_hist_frames < 1) return fail(SA_E_ARG, "sparse_select: no candidate frames");
  if (it.n_hist_frames > it.n_frames_kv)
    return fail(SA_E_RANGE, "sparse_select: n_hist_frames %d > n_frames_kv %d", it.n_hist_frames,
                it.n_frames_kv);
  if (it.n_frames_kv > SA_MAX_FRAMES_KV)
    return fail(SA_E_RANGE, "sparse_select: n_frames_kv %d > %d", it.n_frames_kv, SA_MAX_FRAMES_KV);
  if (it.kv->frame_capacity == 0) return fail(SA_E_RANGE, "sparse_select: the layer has no frames");
  if (it.frames == nullptr) return fail(SA_E_ARG, "sparse_select: frames is NULL");
  const int64_t cand = static_cast<int64_t>(it.n_hist_frames) * ((P + 63) / 64);
  if (cand > kMaxCandidates)
    return fail(SA_E_RANGE, "sparse_select: %lld candidate blocks > %d", static_cast<long long>(cand),
                kMaxCandidates);
  if (it.keep_blocks < 1 || it.keep_blocks > cand)
    return fail(SA_E_ARG, "sparse_select: keep_blocks %d outside [1, %lld]", it.keep_blocks,
                static_cast<long long>(cand));
  a = SelectArgs{};
  fill_item(it, P, a.item);
  a.item.text_window = nullptr;
  a.item.block_list = nullptr;
  a.item.q_tiles = static_cast<int32_t>((rows + SA_SPARSE_QUERY_BLOCK - 1) / SA_SPARSE_QUERY_BLOCK);
  a.heads = geom->heads;
  a.fp8 = it.kv->dtype == SA_KV_FP8_E4M3;
  a.int8 = it.kv->dtype == SA_KV_INT8;
  a.n_cand = static_cast<int32_t>(cand);
  a.keep = it.keep_blocks;
  a.rope = rope_params(geom);
  *ws_bytes = static_cast<size_t>(geom->heads) * static_cast<size_t>(cand) * kD * sizeof(float);
  return ok();
}

// The block-list output of a selection call, and the head bound of its
// selection kernel.
sa_status check_block_list_out(const sa_geom* geom, const int32_t* block_list) {
  if (block_list == nullptr) return fail(SA_E_ARG, "sparse_select: block_list is NULL");
  if ((reinterpret_cast<uintptr_t>(block_list) & 3) != 0)
    return fail(SA_E_ALIGN, "sparse_select: block_list not 4-byte aligned");
  if (geom->heads > 256) return fail(SA_E_SHAPE, "sparse_select: more than 256 heads");
  return SA_OK;
}

}  // namespace

int32_t sa_sparse_keep(int32_t n_candidates, int32_t percent) {
  if (percent < 1 || percent > 100) {
    fail(SA_E_ARG, "sparse_keep: percent %d outside [1, 100]", percent);
    return -1;
  }
  ok();
  if (n_candidates <= 0) return 0;
  const int64_t keep = (static_cast<int64_t>(n_candidates) * percent + 99) / 100;
  return static_cast<int32_t>(std::min<int64_t>(n_candidates, std::max<int64_t>(1, keep)));
}

size_t sa_sparse_select_workspace(const sa_geom* geom, const sa_attn_item* item) {
  SelectArgs a;
  size_t ws = 0;
  if (prepare_select(geom, item, a, &ws) != SA_OK) return 0;
  return ws;
}

sa_status sa_sparse_select(const sa_geom* geom, const sa_attn_item* item, void* workspace,
                           size_t workspace_bytes, int32_t* block_list, void* stream) {
  SelectArgs a;
  size_t ws = 0;
  sa_status st = prepare_select(geom, item, a, &ws);
  if (st != SA_OK) return st;
  if ((st = check_block_list_out(geom, block_list)) != SA_OK) return st;
  if (workspace == nullptr || workspace_bytes < ws)
    return fail(SA_E_CAPACITY, "sparse_select: workspace of %zu bytes < %zu", workspace_bytes, ws);
  if (!aligned16(workspace)) return fail(SA_E_ALIGN, "sparse_select: workspace not 16-byte aligned");
#ifdef SA_DEBUG_CHECKS
  if ((st = debug_check_list(item->frames, item->n_hist_frames, 1, item->kv->frame_capacity, false,
                             static_cast<hipStream_t>(stream), "sparse_select frames")) != SA_OK)
    return st;
#endif
  a.pooled = static_cast<float*>(workspace);
  a.out = block_list;
  return hip_status(launch_sparse_select(a, static_cast<hipStream_t>(stream)), "sparse_select launch");
}

sa_status sa_sparse_select_noalloc(const sa_geom* geom, const sa_attn_item* item,
                                   int32_t* block_list, void* stream) {
  SelectArgs a;
  size_t ws = 0;
  sa_status st = prepare_select(geom, item, a, &ws);
  if (st != SA_OK) return st;
  if ((st = check_block_list_out(geom, block_list)) != SA_OK) return st;
  if (ws > SA_SPARSE_SCRATCH_BYTES)
    return fail(SA_E_CAPACITY,
                "sparse_select_noalloc: %d heads x %d candidate blocks need %zu bytes of pooled "
                "keys > the %u-byte static scratch",
                geom->heads, a.n_cand, ws, SA_SPARSE_SCRATCH_BYTES);
  float* scratch = nullptr;
  if ((st = hip_status(sparse_select_scratch(&scratch), "sparse_select_noalloc scratch address")) !=
      SA_OK)
    return st;
  a.pooled = scratch;
  a.out = block_list;
  return hip_status(launch_sparse_select(a, static_cast<hipStream_t>(stream)),
                    "sparse_select_noalloc launch");
}

sa_status sa_camera_attention(const sa_geom* geom, const void* q, int32_t n_frames,
                              const void* cam_k, const void* cam_v, int32_t n_cam,
                              int32_t kv_heads, int32_t chunk, void* out, float* lse,
                              void* stream) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if (n_frames < 1) return fail(SA_E_ARG, "camera_attention: n_frames %d < 1", n_frames);
  if (chunk < 1 || chunk > SA_MAX_CAMERA_CHUNK)
    return fail(SA_E_ARG, "camera_attention: chunk %d outside [1, %d]", chunk, SA_MAX_CAMERA_CHUNK);
  if (n_cam < n_frames)
    return fail(SA_E_ARG, "camera_attention: %d camera tokens for %d frames", n_cam, n_frames);
  if (kv_heads != 1 && kv_heads != geom->heads)
    return fail(SA_E_ARG, "camera_attention: kv_heads %d is neither 1 nor %d", kv_heads, geom->heads);
  if (q == nullptr || cam_k == nullptr || cam_v == nullptr || out == nullptr)
    return fail(SA_E_ARG, "camera_attention: NULL pointer");
  if (!aligned16(q) || !aligned16(cam_k) || !aligned16(cam_v) || !aligned16(out))
    return fail(SA_E_ALIGN, "camera_attention: pointers not 16-byte aligned");
  const int64_t rows = static_cast<int64_t>(n_frames) * tokens_per_frame(geom);
  if (rows * geom->heads > (int64_t(1) << 31) - 16)
    return fail(SA_E_SHAPE, "camera_attention: too many rows");
  CameraArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.cam_k = static_cast<const uint16_t*>(cam_k);
  a.cam_v = static_cast<const uint16_t*>(cam_v);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.rows = static_cast<int32_t>(rows);
  a.heads = geom->heads;
  a.kv_heads = kv_heads;
  a.P = tokens_per_frame(geom);
  a.n_cam = n_cam;
  a.chunk = chunk;
  const double scale = geom->softmax_scale > 0.f ? geom->softmax_scale : 1.0 / std::sqrt(128.0);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  return hip_status(launch_camera(a, static_cast<hipStream_t>(stream)), "camera_attention launch");
}

sa_status sa_kv_dequant(const sa_geom* geom, const sa_kv_layer* src, const int32_t* d_frames,
                        int32_t n_frames, int32_t n_text, const sa_kv_layer* dst, void* stream) {
  sa_status st = check_geom(geom);
  if (st != SA_OK) return st;
  if ((st = check_layer(geom, src, "dequant src")) != SA_OK) return st;
  if ((st = check_layer(geom, dst, "dequant dst")) != SA_OK) return st;
  if (src->dtype == SA_KV_BF16) return fail(SA_E_UNSUPPORTED, "dequant: src must be fp8 or int8");
  if (dst->dtype != SA_KV_BF16) return fail(SA_E_UNSUPPORTED, "dequant: dst must be bf16");
  if (n_frames < 0 || n_text < 0) return fail(SA_E_ARG, "negative counts");
  if (n_frames > dst->frame_capacity)
    return fail(SA_E_CAPACITY, "dequant: %d frames > dst capacity %d", n_frames, dst->frame_capacity);
  if (n_text > src->text_capacity || n_text > dst->text_capacity)
    return fail(SA_E_CAPACITY, "dequant: n_text %d exceeds a text capacity", n_text);
  if (n_frames > 0 && d_frames == nullptr) return fail(SA_E_ARG, "frames is NULL");
  if (n_frames > 0 && src->frame_capacity == 0) return fail(SA_E_RANGE, "dequant: src has no frames");
  hipStream_t s = static_cast<hipStream_t>(stream);
#ifdef SA_DEBUG_CHECKS
  if ((st = debug_check_list(d_frames, n_frames, 1, src->frame_capacity, false, s,
                             "dequant frames")) != SA_OK)
    return st;
#endif
  if (n_frames > 0) {
    DequantArgs a{};
    a.src_k = static_cast<const uint8_t*>(src->k);
    a.src_v = static_cast<const uint8_t*>(src->v);
    a.src_ks = src->k_scale;
    a.src_vs = src->v_scale;
    a.dst_k = static_cast<uint16_t*>(dst->k);
    a.dst_v = static_cast<uint16_t*>(dst->v);
    a.frames = d_frames;
    a.n = n_frames;
    a.heads = geom->heads;
    a.src_len = frame_slots(geom, src->dtype);
    a.dst_len = a.n_tok = tokens_per_frame(geom);
    a.int8 = src->dtype == SA_KV_INT8;
    if ((st = hip_status(launch_dequant(a, s), "kv_dequant launch")) != SA_OK) return st;
  }
  if (n_text > 0) {
    DequantArgs a{};
    a.src_k = static_cast<const uint8_t*>(src->k_text);
    a.src_v = static_cast<const uint8_t*>(src->v_text);
    a.src_ks = src->k_text_scale;
    a.src_vs = src->v_text_scale;
    a.dst_k = static_cast<uint16_t*>(dst->k_text);
    a.dst_v = static_cast<uint16_t*>(dst->v_text);
    a.frames = nullptr;
    a.n = 1;
    a.heads = geom->heads;
    a.src_len = src->text_capacity;
    a.dst_len = dst->text_capacity;
    a.n_tok = n_text;
    a.int8 = src->dtype == SA_KV_INT8;
    if ((st = hip_status(launch_dequant(a, s), "kv_dequant text launch")) != SA_OK) return st;
  }
  return ok();
}

}  // extern "C"
