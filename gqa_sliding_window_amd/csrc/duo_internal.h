// Internal definitions shared by the host planner and the gfx950 kernels of
// the duo_attn library: kernel parameter blocks, the head-class plan and the
// work-item decoders (host and device use the same functions, so the plan the
// host reports is the plan the kernels execute).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

constexpr int kD = 128;           // head_dim
constexpr int kMaxKv = 32;        // KV heads per layer
constexpr int kMaxGroup = 16;     // query heads per KV head (MFMA columns)
// A prefill workgroup is 4 waves of 32 query rows: 64 rows of two query
// heads of one KV head (even group sizes), else 128 rows of one query head.
constexpr int kPrefillWaveRows = 32;
constexpr int kPrefillWaves = 4;
constexpr int kPrefillKeys = 64;  // keys per prefill K/V tile
// Prefill key-range split: resident prefill workgroups on an MI355X (256 CUs,
// two 4-wave workgroups per CU), the most pieces one unit's keys are cut into,
// the fewest key tiles a piece gets, and the extra cost of a piece (its own
// query load and start-up, its partial write and the merge) in tile-steps.
constexpr int kPrefillSlots = 512;
constexpr int kMaxPieces = 8;
constexpr int kMinPieceTiles = 8;
constexpr int kPieceCost = 4;
// One piece's partial result: [4 waves][2 column blocks][8 dim blocks][64
// lanes] float4 (the unnormalised output in the MFMA accumulator layout),
// then [4 waves][2 column blocks][16 rows] (max, sum) float pairs.
constexpr int kPartOutFloats = 4 * 2 * 8 * 64 * 4;
constexpr int kPartFloats = kPartOutFloats + 4 * 2 * 16 * 2;
constexpr int kDecodeKeys = 32;   // keys per decode tile (one wave)
constexpr int kDecodeWaves = 4;   // waves per decode workgroup
constexpr int kXcds = 8;          // MI355X: 8 XCDs, workgroups dispatched round-robin
// Decode split planning (overridable at build time for tuning sweeps).
#ifndef DUO_DECODE_TARGET_ITEMS
#define DUO_DECODE_TARGET_ITEMS 640       // ~2.5 workgroups per CU
#endif
#ifndef DUO_DECODE_MIN_SPLIT
#define DUO_DECODE_MIN_SPLIT 512          // keys per workgroup, at least 4 tiles per wave
#endif
constexpr int kDecodeTargetItems = DUO_DECODE_TARGET_ITEMS;
constexpr int kDecodeMinSplit = DUO_DECODE_MIN_SPLIT;
constexpr int kDecodeMaxSplits = 256;     // splits of one sequence (bounds the merge)

enum HeadClass : int { kMain = 0, kStream = 1 };

// Head-class plan of one layer (model card "DuoAttention Laguna Adapter",
// "Summary": KV heads are full-context or streaming; "Changes In This
// Submission": heads reordered so the two classes separate). Within a class,
// heads are ranked by ascending KV-head index.
struct HeadPlan {
  int32_t n_main;
  int32_t n_stream;
  uint32_t stream_mask;          // bit kvh set = streaming head
  int8_t main_heads[kMaxKv];     // rank -> kvh
  int8_t stream_heads[kMaxKv];
};

// Index of the n-th set bit of mask (n counted from 0); -1 if there is none.
// Used instead of rank -> head tables so that kernels never index their
// by-value parameter block at run time (which would copy it to scratch).
__host__ __device__ inline int nth_set_bit(uint32_t mask, int n) {
  // (A loop of n steps that clears the lowest set bits, or a branch-free
  // popcount search, changed the code the compiler gave the kernels around
  // it: the 4-token verify block 7% slower, or every prefill and verify
  // block 5-13% slower.)
  for (int b = 0; b < 32; ++b) {
    if ((mask >> b) & 1u) {
      if (n == 0) return b;
      --n;
    }
  }
  return -1;
}

__host__ __device__ inline uint32_t all_heads_mask(int hkv) {
  return hkv >= 32 ? 0xFFFFFFFFu : ((1u << hkv) - 1u);
}

// kv head of the given class and rank
__host__ __device__ inline int class_head(uint32_t stream_mask, int hkv, int cls, int rank) {
  const uint32_t m = cls ? stream_mask : (all_heads_mask(hkv) & ~stream_mask);
  return nth_set_bit(m, rank);
}

__host__ __device__ inline int head_rank(uint32_t stream_mask, int kvh) {
  const uint32_t below = (kvh == 0) ? 0u : (0xFFFFFFFFu >> (32 - kvh));
  const bool s = (stream_mask >> kvh) & 1u;
  return __builtin_popcount((s ? stream_mask : ~stream_mask) & below);
}

// ---------------------------------------------------------------- q/k prologue
// RMSNorm weight and rotary settings applied to q or k rows as they are
// loaded (host-computed turn rates: rotary pair i turns turns[i] times per
// position).
struct QkPrologue {
  const float* norm_w;   // [128] RMSNorm weight, null = no RMSNorm
  float eps;
  int32_t rope;          // 1: rotary embedding on
  float attn_factor;     // multiplies cos and sin
  double turns[kD / 2];
};

inline bool prologue_active(const QkPrologue& pr) { return pr.norm_w != nullptr || pr.rope != 0; }

struct PrologueParams {  // standalone prologue: y = prologue(x), [B, T, H, 128]
  const uint16_t* x;
  uint16_t* y;
  const int32_t* start_pos;  // [B]
  int32_t batch, T, heads;
  QkPrologue pr;
};

// ---------------------------------------------------------------- kv append
struct AppendParams {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* start_pos;
  uint16_t* k_main;
  uint16_t* v_main;
  uint16_t* k_stream;
  uint16_t* v_stream;
  int64_t main_cap;     // slots per (b, head) in the main cache
  int32_t batch, T, hkv;
  int32_t main_ring;    // 1: main cache is a ring of main_cap slots
  int32_t sink, recent;
  int32_t n_main, n_stream;
  uint32_t stream_mask;
  QkPrologue kpro;      // applied to k_new before it is written (inactive: bit copy)
};

// ---------------------------------------------------------------- prefill
struct PrefillParams {
  const uint16_t* q;     // [B, T, Hq, D]
  const uint16_t* k;     // [B, T, Hkv, D]
  const uint16_t* v;
  uint16_t* out;         // [B, T, Hq, D]
  float* lse;            // [B, Hq, T] or null
  const uint16_t* k_main;
  const uint16_t* v_main;
  const uint16_t* k_stream;
  const uint16_t* v_stream;
  int64_t main_cap;
  int64_t start_pos;
  int32_t batch, T, hq, hkv, group;
  int32_t main_window;   // > 0: main-class heads see a causal window of this width
  int32_t main_ring;     // 1: cached main positions live in a ring of main_cap slots
  int32_t sink, recent;
  int32_t n_main, n_stream;
  uint32_t stream_mask;
  int32_t rows;          // query rows per unit: 64 (two query heads per workgroup) or 128 (one)
  int32_t hpw;           // query heads per workgroup: 2 or 1
  int32_t n_qtiles;
  int32_t n_units_main;  // (q tile, batch, main head) units
  int32_t n_units;       // all units
  int32_t n_units_main8; // n_units_main rounded up to a multiple of kXcds
  int32_t n_pieces;      // key-range pieces per main unit (1: no split)
  int32_t* ws_count;     // [n_units_main, group / hpw] arrival counters, zero between calls
  float* ws_part;        // [n_units_main, group / hpw, n_pieces] partial results (kPartFloats each)
  float scale_log2;      // scale * log2(e)
  const float* sink_logits;  // [Hq] attention-sink logits (natural units) or null
  const uint16_t* gate;      // bf16 output gate or null
  int32_t gate_mode;         // 1: gate [B, T, Hq, D]; 2: gate [B, T, Hq]
  int32_t qpro_on;           // apply qpro to the query rows as they are loaded
  QkPrologue qpro;
};

struct PrefillItem {
  int32_t valid;
  int32_t cls;
  int32_t b, kvh, rank, qhead, qtile;
  int32_t unit;   // index of the unit within its class
  int32_t piece;  // key-range piece of a main unit (0 for streaming units)
};

// Workgroup -> work item. Units (one `rows`-row query tile of one KV-head
// group) are ordered main-class units before streaming units. A workgroup
// computes `hpw` consecutive query heads of its unit (qhead is the first). A main
// unit may be cut into n_pieces key-range pieces (long units of a chunked
// prefill over a long past), each a workgroup of its own; its pieces are merged
// by the last one to finish. Unit u runs on XCD u % 8 (workgroups are
// dispatched to XCDs round-robin); the workgroups of the `group` query heads
// of one unit, and its pieces, are consecutive on that XCD, so they share the
// unit's K/V tiles through its L2. When a class's (batch, KV head) groups fill whole 8-wide
// stripes, each XCD takes its groups one at a time, later query tiles first;
// otherwise all groups advance together, later query tiles first, so every
// XCD gets an equal share of each cost level. The main class is padded to a
// multiple of 8 units (padding workgroups exit at once).
// (32-bit arithmetic: the host keeps grids below 2^31 workgroups; a 64-bit
// division would run as a long software sequence in every workgroup.)
__host__ __device__ inline PrefillItem prefill_item(const PrefillParams& p, int block) {
  PrefillItem it{};
  const int x = block % kXcds;
  const int s = block / kXcds;
  const int gw = p.group / p.hpw;           // workgroups per unit and piece
  const int vu = (s / gw) * kXcds + x;      // virtual unit
  const int g = (s % gw) * p.hpw;
  const int main_v = p.n_units_main8 * p.n_pieces;
  int u, n_class;
  if (vu < main_v) {
    const int j = vu / kXcds;
    u = (j / p.n_pieces) * kXcds + x;
    it.piece = j % p.n_pieces;
    if (u >= p.n_units_main) { it.valid = 0; return it; }
    it.cls = kMain;
    n_class = p.n_main;
  } else {
    u = vu - main_v;
    if (u >= p.n_units - p.n_units_main) { it.valid = 0; return it; }
    it.piece = 0;
    it.cls = kStream;
    n_class = p.n_stream;
  }
  it.valid = 1;
  it.unit = u;
  const int groups = p.batch * n_class;
  int grp;
  if (groups % kXcds == 0) {
    // Whole stripes: XCD x = u % 8 walks its own KV groups x, x + 8, ... one
    // after another, each from its last query tile to its first, so the
    // query tiles that share a group's K/V prefix run together in that XCD's
    // L2 (interleaving the groups would need all of them in one L2).
    const int j = u / kXcds;
    grp = (j / p.n_qtiles) * kXcds + u % kXcds;
    it.qtile = p.n_qtiles - 1 - j % p.n_qtiles;
  } else {
    it.qtile = p.n_qtiles - 1 - u / groups;
    grp = u % groups;
  }
  it.b = grp / n_class;
  it.rank = grp % n_class;
  it.kvh = class_head(p.stream_mask, p.hkv, it.cls, it.rank);
  it.qhead = it.kvh * p.group + g;
  return it;
}

// Tiles [t0, t1) of piece `piece` of a unit with `ntiles` key tiles cut into
// n_pieces pieces of ceil(ntiles / n_pieces) tiles; `used` is the number of
// non-empty pieces (the later pieces of a short unit are empty).
struct PieceRange { int t0, t1, used; };
__host__ __device__ inline PieceRange piece_range(int ntiles, int n_pieces, int piece) {
  const int per = (ntiles + n_pieces - 1) / n_pieces;
  PieceRange r;
  if (per == 0) { r.t0 = r.t1 = 0; r.used = 1; return r; }
  r.t0 = piece * per < ntiles ? piece * per : ntiles;
  r.t1 = r.t0 + per < ntiles ? r.t0 + per : ntiles;
  r.used = (ntiles + per - 1) / per;
  return r;
}

// Key ranges (absolute positions, inclusive) a work item must visit for its
// query rows [qa, qb]; span > 0 is the width of a causal band ending at the
// query (window or recent), 0 = no band. Returns the number of ranges (<= 2).
struct KeyRange { int64_t lo, hi; int64_t span; };

__host__ __device__ inline int prefill_key_ranges(const PrefillParams& p, int cls, int64_t qa,
                                                  int64_t qb, KeyRange& r0, KeyRange& r1) {
  if (cls == kMain) {
    const int64_t w = p.main_window;
    r0.lo = (w > 0) ? ((qa - w + 1) > 0 ? (qa - w + 1) : 0) : 0;
    r0.hi = qb;
    r0.span = (w > 0) ? w : 0;
    r1 = r0;
    return 1;
  }
  // streaming head: sink positions [0, sink) that are <= the query, and the
  // `recent` positions ending at the query (model card, "Why It Works").
  KeyRange sink_r{0, (qb < p.sink - 1) ? qb : (int64_t)p.sink - 1, 0};
  int64_t lo = qa - p.recent + 1;
  if (lo < p.sink) lo = p.sink;
  KeyRange recent_r{lo, qb, p.recent};
  const bool has_sink = p.sink > 0;
  const bool has_recent = lo <= qb;
  r0 = has_sink ? sink_r : recent_r;
  r1 = (has_sink && has_recent) ? recent_r : r0;
  return (has_sink ? 1 : 0) + (has_recent ? 1 : 0);
}

__host__ __device__ inline int64_t tiles_of(const KeyRange& r) {
  return r.hi / kPrefillKeys - r.lo / kPrefillKeys + 1;
}

// ---------------------------------------------------------------- decode
struct DecodeParams {
  const uint16_t* q;     // [B, T, Hq, D]
  const int32_t* seq_lens;  // single-token decode: lengths including the query token (its K/V
                            // already appended); block decode: cached lengths before the block
  uint16_t* out;         // [B, T, Hq, D]
  float* lse;            // [B, T, Hq] or null
  const uint16_t* k_main;
  const uint16_t* v_main;
  const uint16_t* k_stream;
  const uint16_t* v_stream;
  const uint16_t* k_new; // block decode: the block's own K/V [B, T, Hkv, D]; null otherwise
  const uint16_t* v_new;
  int32_t* ws_count;     // [B, Hkv, n_cb] arrival counters, zero between calls
  float* ws_ml;          // [B, T, Hq, n_split_max, 2] partial (max, sum)
  float* ws_acc;         // [B, T, Hq, n_split_max, D] partial unnormalised outputs
  int64_t main_cap;      // slots per (b, main head)
  int32_t main_ring;     // main cache is a ring (sliding layer)
  int32_t window;        // sliding layer window (main class), 0 = none
  int32_t batch, hq, hkv, group;
  int32_t sink, recent;
  int32_t n_main, n_stream;
  uint32_t stream_mask;
  int32_t T;             // query tokens per sequence (1 for the single-token decode)
  int32_t n_cb;          // column blocks per work item: 1 (single token, G <= 16 columns) or
                         // ceil(T * G / 32) (block decode: two 16-column MFMA halves per block)
  int32_t split_keys;
  int32_t n_split_main, n_split_stream, n_split_max;
  int32_t n_items_main, n_items;
  float scale_log2;
  const float* sink_logits;  // [Hq] attention-sink logits (natural units) or null
  const uint16_t* gate;      // bf16 output gate or null
  int32_t gate_mode;         // 1: gate [B, T, Hq, D]; 2: gate [B, T, Hq]
  int32_t qpro_on;           // apply qpro to the query rows as they are loaded
  QkPrologue qpro;
};

struct DecodeItem { int32_t cls, b, rank, kvh, split; };

// Work item i: main-class items (batch, head rank, split) first, then
// streaming items.
__host__ __device__ inline DecodeItem decode_item(const DecodeParams& p, int i) {
  DecodeItem it{};
  int ns = p.n_split_main, nc = p.n_main;
  it.cls = kMain;
  if (i >= p.n_items_main) { i -= p.n_items_main; it.cls = kStream; ns = p.n_split_stream; nc = p.n_stream; }
  it.split = i % ns;
  const int bh = i / ns;
  it.b = bh / nc;
  it.rank = bh % nc;
  it.kvh = class_head(p.stream_mask, p.hkv, it.cls, it.rank);
  return it;
}

// Number of cache slots holding visible keys for a sequence of length len:
// every occupied slot is visible to the query at len - 1 (the caches keep
// exactly the positions the visibility rule needs), so a decode reads slots
// [0, n) in storage order.
__host__ __device__ inline int64_t decode_valid_slots(const DecodeParams& p, int cls, int64_t len) {
  // main: a ring of main_cap slots, or a contiguous cache of main_cap >= len
  // slots (the clamp keeps a bad length inside the buffer).
  const int64_t cap = (cls == kStream) ? (int64_t)p.sink + p.recent : p.main_cap;
  return len < cap ? len : cap;
}

// Keys a work item of a (sequence, head) reads: the valid cache slots, then
// (block decode) the block's own T keys, which follow them in this order.
__host__ __device__ inline int64_t decode_keys(const DecodeParams& p, int cls, int64_t len, bool block) {
  return decode_valid_slots(p, cls, len) + (block ? p.T : 0);
}

// Out-of-contract device data recorded by the kernels (bits of
// duo_device_errors). Each kernel file keeps its own word per device; these
// read them (after a device-wide wait) and optionally clear them.
constexpr unsigned kDevAppendPastCapacity = 1u;
constexpr unsigned kDevLengthPastCapacity = 2u;
constexpr unsigned kDevLengthPastPlan = 4u;
hipError_t decode_device_errors(uint32_t* bits, bool clear);
hipError_t append_device_errors(uint32_t* bits, bool clear);

// Launchers (defined in the .hip files).
hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);
hipError_t launch_qk_prologue(const PrologueParams& p, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int64_t n_blocks, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_block(const DecodeParams& p, hipStream_t s);
hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s);
// The library-held decode scratch of duo_attn_decode_noalloc: its size, and
// its address on the current device (resolved once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);

}  // namespace duo
