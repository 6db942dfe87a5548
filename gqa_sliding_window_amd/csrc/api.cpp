// Host side of the duo_attn C ABI: argument validation (synchronous, no side
// effects on error), the head-class and work plans, and kernel launches on the
// caller's stream. See include/duo_attn.h for the contract of every entry.
#include "duo_attn.h"
#include "duo_internal.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

using namespace duo;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DUO_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Positions are int32 on the device side; the kernels form tile and row
// bounds up to a few hundred past the last position (a 256-row query tile,
// 64-key tiles), so the limit keeps a margin below 2^31.
constexpr int64_t kMaxPos = 0x7FFFFFFF - 1024;
constexpr int64_t kMaxGrid = 0x7FFFFFFF;  // workgroups per launch
constexpr int32_t kMaxBlockTokens = 64;   // query tokens per sequence of a block decode

struct Layer {
  int hq, hkv, group, kind, window, sink, recent;
  float scale;
  bool main_ring;     // main cache is a ring of `window` slots
  int main_window;    // causal band of main-class heads (0 = none)
  HeadPlan plan;
};

// Validate a layer description and build its head-class plan (model card
// "DuoAttention Laguna Adapter", "Summary": full-context vs. streaming KV
// heads, one decision per KV head).
int check_layer(const duo_layer* L, Layer* out) {
  if (L == nullptr) return fail(DUO_ERR_INVALID_ARG, "layer is NULL");
  if (L->head_dim != kD) return fail(DUO_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", L->head_dim);
  if (L->num_q_heads <= 0 || L->num_kv_heads <= 0)
    return fail(DUO_ERR_INVALID_ARG, "head counts must be positive (q %d, kv %d)", L->num_q_heads, L->num_kv_heads);
  if (L->num_q_heads % L->num_kv_heads != 0)
    return fail(DUO_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", L->num_q_heads, L->num_kv_heads);
  if (L->num_kv_heads > kMaxKv) return fail(DUO_ERR_UNSUPPORTED, "num_kv_heads %d > %d", L->num_kv_heads, kMaxKv);
  const int group = L->num_q_heads / L->num_kv_heads;
  if (group > DUO_MAX_GROUP) return fail(DUO_ERR_UNSUPPORTED, "group size %d > %d", group, DUO_MAX_GROUP);
  if (L->kind != DUO_LAYER_FULL && L->kind != DUO_LAYER_SLIDING)
    return fail(DUO_ERR_INVALID_ARG, "unknown layer kind %d", L->kind);
  if (L->sink < 0 || L->recent < 0) return fail(DUO_ERR_INVALID_ARG, "sink %d / recent %d must be >= 0", L->sink, L->recent);
  if (!(L->scale >= 0.f) || std::isinf(L->scale)) return fail(DUO_ERR_INVALID_ARG, "scale must be finite and >= 0");
  Layer r{};
  r.hq = L->num_q_heads;
  r.hkv = L->num_kv_heads;
  r.group = group;
  r.kind = L->kind;
  r.window = L->window;
  r.sink = L->sink;
  r.recent = L->recent;
  r.scale = L->scale > 0.f ? L->scale : 1.f / std::sqrt((float)kD);
  r.main_ring = (L->kind == DUO_LAYER_SLIDING && L->window > 0);
  r.main_window = r.main_ring ? L->window : 0;
  std::memset(&r.plan, -1, sizeof(r.plan));
  r.plan.n_main = r.plan.n_stream = 0;
  r.plan.stream_mask = 0;
  for (int h = 0; h < r.hkv; ++h) {
    const bool streaming = L->full_attention_heads != nullptr && L->full_attention_heads[h] == 0;
    if (streaming) {
      r.plan.stream_mask |= 1u << h;
      r.plan.stream_heads[r.plan.n_stream++] = (int8_t)h;
    } else {
      r.plan.main_heads[r.plan.n_main++] = (int8_t)h;
    }
  }
  if (r.plan.n_stream > 0 && r.recent < 1)
    return fail(DUO_ERR_INVALID_ARG, "streaming heads need recent >= 1 (the current token is always kept)");
  if (r.plan.n_stream > 0 && (int64_t)r.sink + r.recent > kMaxPos)
    return fail(DUO_ERR_INVALID_ARG, "sink + recent too large");
  *out = r;
  return DUO_OK;
}

int check_cache(const Layer& L, const duo_kv_cache* c, bool need_main, bool need_stream) {
  if (c == nullptr) return fail(DUO_ERR_INVALID_ARG, "cache is NULL");
  if (need_main && L.plan.n_main > 0) {
    if (c->k_main == nullptr || c->v_main == nullptr) return fail(DUO_ERR_INVALID_ARG, "main cache pointers are NULL");
    if (!aligned16(c->k_main) || !aligned16(c->v_main)) return fail(DUO_ERR_INVALID_ARG, "main cache pointers must be 16-byte aligned");
    if (c->main_capacity <= 0) return fail(DUO_ERR_INVALID_ARG, "main_capacity must be > 0");
    if (L.main_ring && c->main_capacity != L.window)
      return fail(DUO_ERR_INVALID_ARG, "sliding-layer ring must have main_capacity == window (%lld vs %d)",
                  (long long)c->main_capacity, L.window);
  }
  if (need_stream && L.plan.n_stream > 0) {
    if (c->k_stream == nullptr || c->v_stream == nullptr) return fail(DUO_ERR_INVALID_ARG, "stream cache pointers are NULL");
    if (!aligned16(c->k_stream) || !aligned16(c->v_stream)) return fail(DUO_ERR_INVALID_ARG, "stream cache pointers must be 16-byte aligned");
  }
  return DUO_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DUO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Optional q/k prologue: checks the fields and fills the device-side
// settings, including the per-pair turn rates f_i / (2 pi) in double
// precision. f_i = theta^(-2i/128); with YaRN (factor > 1; Peng et al. 2023,
// section 3.2) f_i is blended with f_i / factor by a linear ramp over the pair
// index between floor(c(beta_fast)) and ceil(c(beta_slow)), where c(r) solves
// original_max_position * theta^(-2c/128) = 2 pi r.
int read_prologue(const duo_prologue* e, QkPrologue* pr, int32_t* on) {
  std::memset(pr, 0, sizeof(*pr));
  *on = 0;
  if (e == nullptr) return DUO_OK;
  if (!std::isfinite(e->norm_eps) || e->norm_eps < 0.f) return fail(DUO_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if (e->norm_weight != nullptr && (reinterpret_cast<uintptr_t>(e->norm_weight) & 3u))
    return fail(DUO_ERR_INVALID_ARG, "norm_weight misaligned");
  pr->norm_w = e->norm_weight;
  pr->eps = e->norm_eps;
  if (e->rope != nullptr) {
    const duo_rope& r = *e->rope;
    if (!(r.theta > 1.f) || !std::isfinite(r.theta)) return fail(DUO_ERR_INVALID_ARG, "rope theta must be finite and > 1");
    if (!(r.attention_factor > 0.f) || !std::isfinite(r.attention_factor))
      return fail(DUO_ERR_INVALID_ARG, "rope attention_factor must be finite and > 0");
    if (!(r.factor > 0.f) || !std::isfinite(r.factor)) return fail(DUO_ERR_INVALID_ARG, "rope factor must be finite and > 0");
    const double theta = r.theta;
    const double two_pi = 6.283185307179586476925286766559;
    double low = 0, high = 0;
    const bool yarn = r.factor > 1.f;
    if (yarn) {
      if (r.original_max_position < 1) return fail(DUO_ERR_INVALID_ARG, "original_max_position must be >= 1");
      if (!(r.beta_slow > 0.f) || !(r.beta_fast > r.beta_slow) || !std::isfinite(r.beta_fast))
        return fail(DUO_ERR_INVALID_ARG, "YaRN needs beta_fast > beta_slow > 0");
      auto corr = [&](double turns) {
        return kD * std::log(r.original_max_position / (two_pi * turns)) / (2.0 * std::log(theta));
      };
      low = std::floor(corr(r.beta_fast));
      high = std::ceil(corr(r.beta_slow));
      if (low < 0) low = 0;
      if (high > kD - 1) high = kD - 1;
      if (high == low) high += 0.001;
    }
    for (int i = 0; i < kD / 2; ++i) {
      const double f = std::pow(theta, -2.0 * i / kD);
      double fi = f;
      if (yarn) {
        double ramp = (i - low) / (high - low);
        ramp = ramp < 0 ? 0 : (ramp > 1 ? 1 : ramp);
        fi = f * (1.0 - ramp) + f / r.factor * ramp;
      }
      pr->turns[i] = fi / two_pi;
    }
    pr->rope = 1;
    pr->attn_factor = r.attention_factor;
  }
  *on = prologue_active(*pr) ? 1 : 0;
  return DUO_OK;
}

// Optional epilogue: checks its fields and copies them into the kernel
// parameters (null epilogue = no sink, no gate).
int read_epilogue(const duo_epilogue* e, const float** sink, const uint16_t** gate, int32_t* mode) {
  *sink = nullptr;
  *gate = nullptr;
  *mode = DUO_GATE_NONE;
  if (e == nullptr) return DUO_OK;
  if (e->sink_logits != nullptr && (reinterpret_cast<uintptr_t>(e->sink_logits) & 3u))
    return fail(DUO_ERR_INVALID_ARG, "sink_logits misaligned");
  if (e->gate_mode != DUO_GATE_NONE && e->gate_mode != DUO_GATE_PER_ELEMENT && e->gate_mode != DUO_GATE_PER_HEAD)
    return fail(DUO_ERR_INVALID_ARG, "unknown gate_mode %d", e->gate_mode);
  if ((e->gate != nullptr) != (e->gate_mode != DUO_GATE_NONE))
    return fail(DUO_ERR_INVALID_ARG, "gate and gate_mode must be given together");
  if (e->gate != nullptr && !aligned16(e->gate)) return fail(DUO_ERR_INVALID_ARG, "gate must be 16-byte aligned");
  *sink = e->sink_logits;
  *gate = static_cast<const uint16_t*>(e->gate);
  *mode = e->gate_mode;
  return DUO_OK;
}

// ---- prefill plan
// Key-range pieces per main unit. A long main unit (a chunk's full-context
// query tile over a long past) can outlast the rest of the launch: with few
// such units per resident workgroup slot, the last round of them runs on a
// part of the GPU. When the longest main unit holds more than half the work
// per slot, the plan cuts every main unit into n pieces, n chosen to minimise
// the estimated makespan max(rounds of pieces x piece length, total work /
// slots), each piece costing kPieceCost more tile-steps and holding at least
// kMinPieceTiles key tiles; otherwise n = 1.
int choose_pieces(const PrefillParams& p) {
  if (p.n_main == 0 || p.n_qtiles > 65536) return 1;
  int64_t wm = 0, ws = 0, lmax = 0;
  const int64_t last = p.start_pos + p.T - 1;
  for (int qt = 0; qt < p.n_qtiles; ++qt) {
    const int64_t qa = p.start_pos + (int64_t)qt * p.rows;
    const int64_t qb = qa + p.rows - 1 < last ? qa + p.rows - 1 : last;
    KeyRange r0, r1;
    prefill_key_ranges(p, kMain, qa, qb, r0, r1);
    const int64_t nm = tiles_of(r0);
    wm += nm;
    lmax = nm > lmax ? nm : lmax;
    if (p.n_stream > 0) {
      const int nr = prefill_key_ranges(p, kStream, qa, qb, r0, r1);
      ws += (nr > 0 ? tiles_of(r0) : 0) + (nr > 1 ? tiles_of(r1) : 0);
    }
  }
  const int64_t gw = p.group / p.hpw;  // workgroups per unit
  const int64_t per_qt_main = (int64_t)p.batch * p.n_main * gw;  // workgroups per query tile
  const int64_t total = (wm * p.n_main + ws * p.n_stream) * p.batch * gw;
  const int64_t nm_wg = per_qt_main * p.n_qtiles;
  if (lmax * 2 * kPrefillSlots <= total) return 1;
  auto est = [&](int n) {
    const int64_t rounds = (nm_wg * n + kPrefillSlots - 1) / kPrefillSlots;
    const int64_t piece = (lmax + n - 1) / n + (n > 1 ? kPieceCost : 0);
    const int64_t spread = (total + (n > 1 ? nm_wg * n * kPieceCost : 0)) / kPrefillSlots;
    return rounds * piece > spread ? rounds * piece : spread;
  };
  int best = 1;
  int64_t best_est = est(1);
  for (int n = 2; n <= kMaxPieces && lmax >= (int64_t)n * kMinPieceTiles; ++n) {
    const int64_t e = est(n);
    if (e * 50 < best_est * 49) {  // at least 2% better
      best = n;
      best_est = e;
    }
  }
  return best;
}

// split = false: every unit in one workgroup (no workspace); true: the
// key-range pieces of choose_pieces.
int build_prefill(const Layer& L, int32_t batch, int32_t T, int64_t start_pos, bool split, PrefillParams* p,
                  int64_t* n_blocks) {
  std::memset(p, 0, sizeof(*p));
  p->start_pos = start_pos;
  p->batch = batch;
  p->T = T;
  p->hq = L.hq;
  p->hkv = L.hkv;
  p->group = L.group;
  p->main_window = L.main_window;
  p->main_ring = L.main_ring ? 1 : 0;
  p->sink = L.sink;
  p->recent = L.recent;
  p->n_main = L.plan.n_main;
  p->n_stream = L.plan.n_stream;
  p->stream_mask = L.plan.stream_mask;
  p->hpw = (L.group % 2 == 0) ? 2 : 1;
  p->rows = kPrefillWaves * kPrefillWaveRows / p->hpw;
  p->n_qtiles = (T + p->rows - 1) / p->rows;
  const int64_t um = (int64_t)p->n_qtiles * batch * L.plan.n_main;
  const int64_t us = (int64_t)p->n_qtiles * batch * L.plan.n_stream;
  if (um + us + kXcds > kMaxGrid / kMaxPieces) return fail(DUO_ERR_INVALID_ARG, "prefill work too large for one launch");
  p->n_units_main = (int32_t)um;
  p->n_units = (int32_t)(um + us);
  p->n_units_main8 = (int32_t)((um + kXcds - 1) / kXcds * kXcds);
  p->n_pieces = split ? choose_pieces(*p) : 1;
  p->scale_log2 = L.scale * 1.4426950408889634f;
  const int64_t virt = (int64_t)p->n_units_main8 * p->n_pieces + us;
  const int64_t units8 = (virt + kXcds - 1) / kXcds * kXcds;
  *n_blocks = units8 * (L.group / p->hpw);
  if (*n_blocks > kMaxGrid) return fail(DUO_ERR_INVALID_ARG, "prefill grid too large");
  return DUO_OK;
}

// Prefill workspace: one slot per (main unit, workgroup of the unit): [slots]
// int32 arrival counters | [slots * n_pieces] partial results of kPartFloats
// floats; both parts 256-byte aligned. Empty without pieces.
struct PrefillWs { size_t part, total; };

PrefillWs prefill_ws_layout(const PrefillParams& p) {
  PrefillWs w{0, 0};
  if (p.n_pieces <= 1) return w;
  const size_t slots = (size_t)p.n_units_main * (p.group / p.hpw);
  w.part = (slots * sizeof(int32_t) + 255) / 256 * 256;
  w.total = w.part + slots * p.n_pieces * (size_t)kPartFloats * sizeof(float);
  return w;
}

// ---- decode plan: keys per workgroup split chosen so the launch has about
// kDecodeTargetItems workgroups, a multiple of one tile per wave, never fewer
// than kDecodeMinSplit keys and never more than kDecodeMaxSplits splits of one
// sequence.
// block_tokens = 0: single-token decode (the query's K/V already in the
// cache); > 0: block decode of that many tokens after the max_seq_len cached
// positions (their K/V read from the call's inputs).
int build_decode(const Layer& L, int32_t batch, int64_t max_seq_len, int64_t main_cap, DecodeParams* p,
                 int32_t block_tokens = 0) {
  std::memset(p, 0, sizeof(*p));
  p->batch = batch;
  p->hq = L.hq;
  p->hkv = L.hkv;
  p->group = L.group;
  p->main_ring = L.main_ring ? 1 : 0;
  p->main_cap = main_cap;
  p->sink = L.sink;
  p->recent = L.recent;
  p->n_main = L.plan.n_main;
  p->n_stream = L.plan.n_stream;
  p->stream_mask = L.plan.stream_mask;
  p->scale_log2 = L.scale * 1.4426950408889634f;
  p->window = L.main_ring ? L.window : 0;
  p->T = block_tokens > 0 ? block_tokens : 1;
  // column blocks per work item: 16 columns (one MFMA width) for the
  // single-token decode; for a block, one block of at most 32 (T G) columns,
  // else blocks of 48 (each workgroup streams the item's keys once for its
  // columns)
  p->n_cb = block_tokens > 0 ? (p->T * L.group <= 32 ? 1 : (p->T * L.group + 47) / 48) : (L.group + 15) / 16;
  const int64_t extra = block_tokens;  // the block's own keys follow the cached ones
  const int64_t keys_main = (L.main_ring ? (max_seq_len < L.window ? max_seq_len : L.window) : max_seq_len) + extra;
  const int64_t sr = (int64_t)L.sink + L.recent;
  const int64_t keys_stream = (max_seq_len < sr ? max_seq_len : sr) + extra;
  const int64_t total = (int64_t)batch * (L.plan.n_main * keys_main + L.plan.n_stream * keys_stream);
  const int64_t unit = (int64_t)kDecodeKeys * kDecodeWaves;
  // (a block decode launches n_cb workgroups per item: the target counts workgroups)
  const int64_t target = kDecodeTargetItems / p->n_cb > 8 ? kDecodeTargetItems / p->n_cb : 8;
  int64_t split = (total + target - 1) / target;
  if (split < kDecodeMinSplit) split = kDecodeMinSplit;
  const int64_t longest = keys_main > keys_stream ? keys_main : keys_stream;
  const int64_t min_for_cap = (longest + kDecodeMaxSplits - 1) / kDecodeMaxSplits;
  if (split < min_for_cap) split = min_for_cap;
  split = (split + unit - 1) / unit * unit;
  if (split > kMaxPos) split = kMaxPos / unit * unit;
  p->split_keys = (int32_t)split;
  p->n_split_main = L.plan.n_main > 0 ? (int32_t)((keys_main + split - 1) / split) : 0;
  p->n_split_stream = L.plan.n_stream > 0 ? (int32_t)((keys_stream + split - 1) / split) : 0;
  if (p->n_split_main < 1 && L.plan.n_main > 0) p->n_split_main = 1;
  if (p->n_split_stream < 1 && L.plan.n_stream > 0) p->n_split_stream = 1;
  p->n_split_max = p->n_split_main > p->n_split_stream ? p->n_split_main : p->n_split_stream;
  const int64_t im = (int64_t)batch * L.plan.n_main * p->n_split_main;
  const int64_t is = (int64_t)batch * L.plan.n_stream * p->n_split_stream;
  if ((im + is + kXcds) * p->n_cb > kMaxGrid) return fail(DUO_ERR_INVALID_ARG, "decode work too large for one launch");
  p->n_items_main = (int32_t)im;
  p->n_items = (int32_t)(im + is);
  return DUO_OK;
}

// Workspace: [B * Hkv * column blocks] int32 arrival counters |
// [B, T, Hq, splits, 2] partial (max, sum) | [B, T, Hq, splits, 128] partial
// outputs; each part 256-byte aligned.
struct WsLayout { size_t count, ml, acc, total; };

WsLayout decode_ws_layout(const DecodeParams& p) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t n = (size_t)p.batch * p.T * p.hq * (size_t)p.n_split_max;
  WsLayout w;
  w.count = 0;
  w.ml = up((size_t)p.batch * p.hkv * p.n_cb * sizeof(int32_t));
  w.acc = w.ml + up(n * 2 * sizeof(float));
  w.total = w.acc + n * kD * sizeof(float);
  return w;
}

size_t decode_ws_bytes(const DecodeParams& p) { return decode_ws_layout(p).total; }

}  // namespace

extern "C" {

int duo_attn_version(void) { return DUO_ATTN_VERSION; }

int duo_prefill_tile_rows(const duo_layer* layer) {
  Layer L;
  const int rc = check_layer(layer, &L);
  if (rc) return rc;
  ok();
  return kPrefillWaves * kPrefillWaveRows / (L.group % 2 == 0 ? 2 : 1);
}

const char* duo_last_error(void) { return g_err; }

int duo_device_errors(uint32_t* bits, int32_t clear) {
  static_assert(kDevAppendPastCapacity == DUO_DEVICE_APPEND_PAST_CAPACITY &&
                    kDevLengthPastCapacity == DUO_DEVICE_LENGTH_PAST_CAPACITY &&
                    kDevLengthPastPlan == DUO_DEVICE_LENGTH_PAST_PLAN,
                "device error bits match the header");
  if (bits == nullptr) return fail(DUO_ERR_INVALID_ARG, "bits is NULL");
  uint32_t v = 0u;
  int rc = hip_status(hipDeviceSynchronize(), "device wait");
  if (rc) return rc;
  rc = hip_status(decode_device_errors(&v, clear != 0), "decode error word");
  if (rc) return rc;
  rc = hip_status(append_device_errors(&v, clear != 0), "append error word");
  if (rc) return rc;
  *bits = v;
  return ok();
}

int duo_head_plan(const duo_layer* layer, int32_t* head_class, int32_t* head_rank_out, int32_t* n_main,
                  int32_t* n_stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  for (int h = 0; h < L.hkv; ++h) {
    const bool s = (L.plan.stream_mask >> h) & 1u;
    if (head_class) head_class[h] = s ? 1 : 0;
    if (head_rank_out) head_rank_out[h] = head_rank(L.plan.stream_mask, h);
  }
  if (n_main) *n_main = L.plan.n_main;
  if (n_stream) *n_stream = L.plan.n_stream;
  return ok();
}

int duo_kv_cache_bytes(const duo_layer* layer, int32_t batch, int64_t capacity, int64_t* main_bytes,
                       int64_t* stream_bytes) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0 || capacity < 0) return fail(DUO_ERR_INVALID_ARG, "batch and capacity must be >= 0");
  const int64_t main_slots = L.main_ring ? L.window : capacity;
  const int64_t row = kD * 2;
  if (main_bytes) *main_bytes = (int64_t)batch * L.plan.n_main * main_slots * row;
  if (stream_bytes) *stream_bytes = (int64_t)batch * L.plan.n_stream * ((int64_t)L.sink + L.recent) * row;
  return ok();
}

int duo_kv_cache_report(const duo_layer* layer, int32_t batch, int64_t capacity, const int32_t* seq_lens,
                        duo_cache_report* out) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0 || capacity < 0) return fail(DUO_ERR_INVALID_ARG, "batch and capacity must be >= 0");
  if (out == nullptr || (batch > 0 && seq_lens == nullptr)) return fail(DUO_ERR_INVALID_ARG, "NULL argument");
  const int64_t main_per_head = L.main_ring ? L.window : capacity;
  const int64_t stream_per_head = (int64_t)L.sink + L.recent;
  const int64_t slot_bytes = 2 * kD * 2;  // K and V rows of one slot
  std::memset(out, 0, sizeof(*out));
  out->main_slots = (int64_t)batch * L.plan.n_main * main_per_head;
  out->stream_slots = (int64_t)batch * L.plan.n_stream * stream_per_head;
  out->base_slots = (int64_t)batch * L.hkv * main_per_head;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = seq_lens[b] > 0 ? seq_lens[b] : 0;
    out->main_active += L.plan.n_main * std::min(len, main_per_head);
    out->stream_active += L.plan.n_stream * std::min(len, stream_per_head);
    out->base_active += L.hkv * std::min(len, main_per_head);
  }
  out->main_bytes = out->main_slots * slot_bytes;
  out->stream_bytes = out->stream_slots * slot_bytes;
  out->base_bytes = out->base_slots * slot_bytes;
  return ok();
}

int duo_kv_append(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch, const void* k_new,
                  const void* v_new, int32_t num_tokens, const int32_t* start_pos, int64_t max_end_pos,
                  const duo_prologue* k_prologue, void* stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0 || num_tokens < 0) return fail(DUO_ERR_INVALID_ARG, "batch and num_tokens must be >= 0");
  if (batch == 0 || num_tokens == 0) return ok();
  if ((rc = check_cache(L, cache, true, true))) return rc;
  if (k_new == nullptr || v_new == nullptr || start_pos == nullptr)
    return fail(DUO_ERR_INVALID_ARG, "k_new, v_new and start_pos must not be NULL");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(DUO_ERR_INVALID_ARG, "k_new/v_new must be 16-byte aligned");
  if (max_end_pos < num_tokens || max_end_pos > kMaxPos)
    return fail(DUO_ERR_INVALID_ARG, "max_end_pos %lld out of range", (long long)max_end_pos);
  if (L.plan.n_main > 0 && !L.main_ring && max_end_pos > cache->main_capacity)
    return fail(DUO_ERR_CAPACITY, "positions up to %lld exceed main_capacity %lld", (long long)max_end_pos,
                (long long)cache->main_capacity);
  if ((int64_t)batch * num_tokens * L.hkv / 16 + 1 > kMaxGrid) return fail(DUO_ERR_INVALID_ARG, "append too large");
  AppendParams p{};
  int32_t pro_on = 0;
  if ((rc = read_prologue(k_prologue, &p.kpro, &pro_on))) return rc;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.start_pos = start_pos;
  p.k_main = static_cast<uint16_t*>(cache->k_main);
  p.v_main = static_cast<uint16_t*>(cache->v_main);
  p.k_stream = static_cast<uint16_t*>(cache->k_stream);
  p.v_stream = static_cast<uint16_t*>(cache->v_stream);
  p.main_cap = cache->main_capacity;
  p.batch = batch;
  p.T = num_tokens;
  p.hkv = L.hkv;
  p.main_ring = L.main_ring ? 1 : 0;
  p.sink = L.sink;
  p.recent = L.recent;
  p.n_main = L.plan.n_main;
  p.n_stream = L.plan.n_stream;
  p.stream_mask = L.plan.stream_mask;
  return hip_status(launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv_append launch");
}

int duo_prefill_plan(const duo_layer* layer, int32_t batch, int32_t num_tokens, int64_t start_pos,
                     int32_t with_workspace, int32_t* items, int64_t* n_items) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0 || num_tokens < 0 || start_pos < 0) return fail(DUO_ERR_INVALID_ARG, "negative size");
  if (start_pos + num_tokens > kMaxPos) return fail(DUO_ERR_INVALID_ARG, "positions exceed %lld", (long long)kMaxPos);
  PrefillParams p;
  int64_t nb = 0;
  if (batch > 0 && num_tokens > 0 &&
      (rc = build_prefill(L, batch, num_tokens, start_pos, with_workspace != 0, &p, &nb)))
    return rc;
  if (n_items) *n_items = nb;
  if (items) {
    for (int64_t i = 0; i < nb; ++i) {
      const PrefillItem it = prefill_item(p, (int)i);
      int32_t* o = items + 7 * i;
      o[0] = o[1] = o[2] = -1;
      o[3] = o[4] = o[5] = o[6] = 0;
      if (!it.valid) continue;
      const int64_t qa = start_pos + (int64_t)it.qtile * p.rows;
      const int64_t last = start_pos + num_tokens - 1;
      const int64_t qb = qa + p.rows - 1 < last ? qa + p.rows - 1 : last;
      KeyRange r0, r1;
      const int nr = prefill_key_ranges(p, it.cls, qa, qb, r0, r1);
      const int64_t tiles = tiles_of(r0) + (nr > 1 ? tiles_of(r1) : 0);
      const PieceRange pr = piece_range((int)tiles, it.cls == kMain ? p.n_pieces : 1, it.piece);
      o[0] = it.b; o[1] = it.qhead; o[2] = it.qtile; o[3] = pr.t1 - pr.t0; o[4] = it.piece; o[5] = pr.used;
      o[6] = p.hpw;
    }
  }
  return ok();
}

size_t duo_attn_prefill_workspace_bytes(const duo_layer* layer, int32_t batch, int32_t num_tokens,
                                        int64_t start_pos) {
  Layer L;
  if (check_layer(layer, &L)) return 0;
  if (batch <= 0 || num_tokens <= 0 || start_pos < 0 || start_pos + num_tokens > kMaxPos) return 0;
  PrefillParams p;
  int64_t nb = 0;
  if (build_prefill(L, batch, num_tokens, start_pos, true, &p, &nb)) return 0;
  ok();
  return prefill_ws_layout(p).total;
}

int duo_attn_prefill(const duo_layer* layer, const duo_kv_cache* past, int32_t batch, const void* q,
                     const void* k, const void* v, int32_t num_tokens, int64_t start_pos, void* out,
                     float* lse, void* workspace, size_t workspace_bytes, const duo_prologue* q_prologue,
                     const duo_epilogue* epilogue, void* stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0 || num_tokens < 0 || start_pos < 0) return fail(DUO_ERR_INVALID_ARG, "negative size or start_pos");
  if (start_pos + num_tokens > kMaxPos) return fail(DUO_ERR_INVALID_ARG, "positions exceed %lld", (long long)kMaxPos);
  if (batch == 0 || num_tokens == 0) return ok();
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr)
    return fail(DUO_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(DUO_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(DUO_ERR_INVALID_ARG, "lse misaligned");
  duo_kv_cache none{};
  if (start_pos > 0) {
    if (past == nullptr) return fail(DUO_ERR_INVALID_ARG, "start_pos > 0 needs the past cache");
    if ((rc = check_cache(L, past, true, true))) return rc;
    if (L.plan.n_main > 0 && !L.main_ring && start_pos > past->main_capacity)
      return fail(DUO_ERR_CAPACITY, "start_pos %lld exceeds main_capacity %lld", (long long)start_pos,
                  (long long)past->main_capacity);
  } else {
    past = past ? past : &none;
  }
  PrefillParams p;
  int64_t nb = 0;
  if ((rc = build_prefill(L, batch, num_tokens, start_pos, workspace != nullptr, &p, &nb))) return rc;
  const PrefillWs wl = prefill_ws_layout(p);
  if (workspace != nullptr) {
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(DUO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (workspace_bytes < wl.total)
      return fail(DUO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total, workspace_bytes);
    p.ws_count = static_cast<int32_t*>(workspace);
    p.ws_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.part);
  }
  if ((rc = read_epilogue(epilogue, &p.sink_logits, &p.gate, &p.gate_mode))) return rc;
  if ((rc = read_prologue(q_prologue, &p.qpro, &p.qpro_on))) return rc;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.k_main = static_cast<const uint16_t*>(past->k_main);
  p.v_main = static_cast<const uint16_t*>(past->v_main);
  p.k_stream = static_cast<const uint16_t*>(past->k_stream);
  p.v_stream = static_cast<const uint16_t*>(past->v_stream);
  p.main_cap = L.main_ring ? L.window : (past->main_capacity > 0 ? past->main_capacity : 1);
  return hip_status(launch_prefill(p, nb, static_cast<hipStream_t>(stream)), "prefill launch");
}

size_t duo_attn_decode_workspace_bytes(const duo_layer* layer, int32_t batch, int64_t max_seq_len) {
  Layer L;
  if (check_layer(layer, &L)) return 0;
  if (batch <= 0 || max_seq_len <= 0 || max_seq_len > kMaxPos) return 0;
  DecodeParams p;
  if (build_decode(L, batch, max_seq_len, L.main_ring ? L.window : max_seq_len, &p)) return 0;
  ok();
  return decode_ws_bytes(p);
}

int duo_decode_plan(const duo_layer* layer, int32_t batch, int64_t max_seq_len, int32_t* split_keys,
                    int32_t* items, int64_t* n_items) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch <= 0 || max_seq_len <= 0 || max_seq_len > kMaxPos) return fail(DUO_ERR_INVALID_ARG, "bad batch or max_seq_len");
  DecodeParams p;
  if ((rc = build_decode(L, batch, max_seq_len, L.main_ring ? L.window : max_seq_len, &p))) return rc;
  if (split_keys) *split_keys = p.split_keys;
  if (n_items) *n_items = p.n_items;
  if (items) {
    for (int64_t i = 0; i < p.n_items; ++i) {
      const DecodeItem it = decode_item(p, (int)i);
      int32_t* o = items + 4 * i;
      o[0] = it.b; o[1] = it.kvh; o[2] = it.split; o[3] = it.cls;
    }
  }
  return ok();
}

}  // extern "C"

namespace {

// Validation and parameters shared by duo_attn_decode and
// duo_attn_decode_noalloc (everything but the workspace).
int prepare_decode(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch, const void* q,
                   const int32_t* seq_lens, int64_t max_seq_len, void* out, float* lse,
                   const duo_prologue* q_prologue, const duo_epilogue* epilogue, DecodeParams* p) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (max_seq_len <= 0 || max_seq_len > kMaxPos) return fail(DUO_ERR_INVALID_ARG, "max_seq_len out of range");
  if (q == nullptr || seq_lens == nullptr || out == nullptr) return fail(DUO_ERR_INVALID_ARG, "q, seq_lens and out must not be NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(DUO_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(DUO_ERR_INVALID_ARG, "lse misaligned");
  if ((rc = check_cache(L, cache, true, true))) return rc;
  if (L.plan.n_main > 0 && !L.main_ring && max_seq_len > cache->main_capacity)
    return fail(DUO_ERR_CAPACITY, "max_seq_len %lld exceeds main_capacity %lld", (long long)max_seq_len,
                (long long)cache->main_capacity);
  const int64_t main_cap = L.main_ring ? L.window : (L.plan.n_main > 0 ? cache->main_capacity : 1);
  if ((rc = build_decode(L, batch, max_seq_len, main_cap, p))) return rc;
  if ((rc = read_epilogue(epilogue, &p->sink_logits, &p->gate, &p->gate_mode))) return rc;
  if ((rc = read_prologue(q_prologue, &p->qpro, &p->qpro_on))) return rc;
  p->q = static_cast<const uint16_t*>(q);
  p->seq_lens = seq_lens;
  p->out = static_cast<uint16_t*>(out);
  p->lse = lse;
  p->k_main = static_cast<const uint16_t*>(cache->k_main);
  p->v_main = static_cast<const uint16_t*>(cache->v_main);
  p->k_stream = static_cast<const uint16_t*>(cache->k_stream);
  p->v_stream = static_cast<const uint16_t*>(cache->v_stream);
  return DUO_OK;
}

void attach_decode_ws(DecodeParams* p, void* workspace) {
  const WsLayout wl = decode_ws_layout(*p);
  char* ws = static_cast<char*>(workspace);
  p->ws_count = reinterpret_cast<int32_t*>(ws + wl.count);
  p->ws_ml = reinterpret_cast<float*>(ws + wl.ml);
  p->ws_acc = reinterpret_cast<float*>(ws + wl.acc);
}

}  // namespace

extern "C" {

int duo_attn_decode(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch, const void* q,
                    const int32_t* seq_lens, int64_t max_seq_len, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, const duo_prologue* q_prologue, const duo_epilogue* epilogue,
                    void* stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0) return fail(DUO_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  DecodeParams p;
  rc = prepare_decode(layer, cache, batch, q, seq_lens, max_seq_len, out, lse, q_prologue, epilogue, &p);
  if (rc) return rc;
  const size_t need = decode_ws_bytes(p);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DUO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DUO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  attach_decode_ws(&p, workspace);
  return hip_status(launch_decode(p, static_cast<hipStream_t>(stream)), "decode launch");
}

int duo_attn_decode_noalloc(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch, const void* q,
                            const int32_t* seq_lens, int64_t max_seq_len, void* out, float* lse,
                            const duo_prologue* q_prologue, const duo_epilogue* epilogue, void* stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0) return fail(DUO_ERR_INVALID_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  DecodeParams p;
  rc = prepare_decode(layer, cache, batch, q, seq_lens, max_seq_len, out, lse, q_prologue, epilogue, &p);
  if (rc) return rc;
  const size_t need = decode_ws_bytes(p);
  if (need > noalloc_scratch_bytes())
    return fail(DUO_ERR_WORKSPACE, "this decode needs %zu bytes of scratch; the library holds %zu (use duo_attn_decode)",
                need, noalloc_scratch_bytes());
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if ((rc = hip_status(noalloc_scratch(&scratch), "decode scratch"))) return rc;
  attach_decode_ws(&p, scratch);
  // the arrival counters start at zero on every call (a fill kernel, not a
  // memset: safe under graph capture)
  const int64_t counters = (int64_t)p.batch * p.hkv * p.n_cb;
  if ((rc = hip_status(launch_fill_zero(p.ws_count, counters, s), "decode scratch clear"))) return rc;
  return hip_status(launch_decode(p, s), "decode launch");
}

size_t duo_attn_decode_block_workspace_bytes(const duo_layer* layer, int32_t batch, int32_t num_tokens,
                                             int64_t max_past_len) {
  Layer L;
  if (check_layer(layer, &L)) return 0;
  if (batch <= 0 || num_tokens < 1 || num_tokens > kMaxBlockTokens || max_past_len < 0 ||
      max_past_len + num_tokens > kMaxPos)
    return 0;
  DecodeParams p;
  if (build_decode(L, batch, max_past_len, L.main_ring ? L.window : (max_past_len > 0 ? max_past_len : 1), &p,
                   num_tokens))
    return 0;
  ok();
  return decode_ws_bytes(p);
}

int duo_attn_decode_block(const duo_layer* layer, const duo_kv_cache* cache, int32_t batch, const void* q,
                          const void* k_new, const void* v_new, int32_t num_tokens, const int32_t* past_lens,
                          int64_t max_past_len, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          const duo_prologue* q_prologue, const duo_epilogue* epilogue, void* stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if (batch < 0) return fail(DUO_ERR_INVALID_ARG, "batch must be >= 0");
  if (num_tokens < 1 || num_tokens > kMaxBlockTokens)
    return fail(DUO_ERR_INVALID_ARG, "num_tokens must be in [1, %d]", kMaxBlockTokens);
  if (batch == 0) return ok();
  if (max_past_len < 0 || max_past_len + num_tokens > kMaxPos) return fail(DUO_ERR_INVALID_ARG, "max_past_len out of range");
  if (q == nullptr || k_new == nullptr || v_new == nullptr || past_lens == nullptr || out == nullptr)
    return fail(DUO_ERR_INVALID_ARG, "q, k_new, v_new, past_lens and out must not be NULL");
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
    return fail(DUO_ERR_INVALID_ARG, "q, k_new, v_new and out must be 16-byte aligned");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(DUO_ERR_INVALID_ARG, "lse misaligned");
  if ((rc = check_cache(L, cache, true, true))) return rc;
  if (L.plan.n_main > 0 && !L.main_ring && max_past_len > cache->main_capacity)
    return fail(DUO_ERR_CAPACITY, "max_past_len %lld exceeds main_capacity %lld", (long long)max_past_len,
                (long long)cache->main_capacity);
  DecodeParams p;
  const int64_t main_cap = L.main_ring ? L.window : (L.plan.n_main > 0 ? cache->main_capacity : 1);
  if ((rc = build_decode(L, batch, max_past_len, main_cap, &p, num_tokens))) return rc;
  const size_t need = decode_ws_bytes(p);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DUO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DUO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if ((rc = read_epilogue(epilogue, &p.sink_logits, &p.gate, &p.gate_mode))) return rc;
  if ((rc = read_prologue(q_prologue, &p.qpro, &p.qpro_on))) return rc;
  p.q = static_cast<const uint16_t*>(q);
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.seq_lens = past_lens;
  p.out = static_cast<uint16_t*>(out);
  p.lse = lse;
  p.k_main = static_cast<const uint16_t*>(cache->k_main);
  p.v_main = static_cast<const uint16_t*>(cache->v_main);
  p.k_stream = static_cast<const uint16_t*>(cache->k_stream);
  p.v_stream = static_cast<const uint16_t*>(cache->v_stream);
  const WsLayout wl = decode_ws_layout(p);
  char* ws = static_cast<char*>(workspace);
  p.ws_count = reinterpret_cast<int32_t*>(ws + wl.count);
  p.ws_ml = reinterpret_cast<float*>(ws + wl.ml);
  p.ws_acc = reinterpret_cast<float*>(ws + wl.acc);
  return hip_status(launch_decode_block(p, static_cast<hipStream_t>(stream)), "decode block launch");
}

int duo_attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr) return fail(DUO_ERR_INVALID_ARG, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return fail(DUO_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return hip_status(launch_fill_zero(static_cast<int32_t*>(workspace), (int64_t)(workspace_bytes / 4),
                                     static_cast<hipStream_t>(stream)),
                    "workspace init launch");
}

int duo_rope_frequencies(const duo_rope* rope, double* freqs) {
  if (rope == nullptr || freqs == nullptr) return fail(DUO_ERR_INVALID_ARG, "rope and freqs must not be NULL");
  duo_prologue e{nullptr, 0.f, rope};
  QkPrologue pr;
  int32_t on = 0;
  const int rc = read_prologue(&e, &pr, &on);
  if (rc) return rc;
  for (int i = 0; i < kD / 2; ++i) freqs[i] = pr.turns[i] * 6.283185307179586476925286766559;
  return ok();
}

int duo_qk_prologue(const duo_prologue* prologue, int32_t batch, int32_t num_tokens, int32_t heads,
                    const void* x, void* y, const int32_t* start_pos, void* stream) {
  if (batch < 0 || num_tokens < 0 || heads < 1 || heads > 4096)
    return fail(DUO_ERR_INVALID_ARG, "batch, num_tokens must be >= 0 and heads in [1, 4096]");
  if (prologue == nullptr) return fail(DUO_ERR_INVALID_ARG, "prologue is NULL");
  PrologueParams p{};
  int32_t on = 0;
  int rc = read_prologue(prologue, &p.pr, &on);
  if (rc) return rc;
  if (batch == 0 || num_tokens == 0) return ok();
  if (x == nullptr || y == nullptr || start_pos == nullptr) return fail(DUO_ERR_INVALID_ARG, "x, y and start_pos must not be NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(DUO_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  if ((int64_t)batch * num_tokens * heads / 32 + 1 > kMaxGrid) return fail(DUO_ERR_INVALID_ARG, "prologue too large");
  p.x = static_cast<const uint16_t*>(x);
  p.y = static_cast<uint16_t*>(y);
  p.start_pos = start_pos;
  p.batch = batch;
  p.T = num_tokens;
  p.heads = heads;
  return hip_status(launch_qk_prologue(p, static_cast<hipStream_t>(stream)), "qk prologue launch");
}

}  // extern "C"
