// Decode attention kernel (gfx950): split-K over the KV cache with the merge
// of partial softmax states done in the same launch.
//
// One query token per sequence at position L-1 (its K/V already appended).
// Full-context heads read every cached position, streaming heads read their
// sink + recent slots (model card "DuoAttention Laguna Adapter", "Why It
// Works": a streaming head holds only the sequence's first positions and its
// newest ones),
// a sliding layer reads its window ring (Laguna-M.1-8bit blog post,
// sliding-window section). Every occupied slot of a cache is visible to the
// decode query, so a decode reads slots [0, n) in storage order; softmax does
// not depend on key order.
//
// Workgroup = 4 waves = one (sequence, KV head, split). The G query heads of
// the KV head are the 16 MFMA columns (G <= 16): one pass over K/V serves the
// whole group. Each wave streams its own interleaved 32-key tiles (16-byte
// coalesced loads, two tiles ahead in registers, a wave-private LDS tile for
// the MFMA operand layouts: K row-major, V read transposed) and keeps its own
// running (max, sum, output); the waves are combined through LDS.
// The block decode (T query tokens per sequence, attend then append) uses
// the same body with (token, head) columns: up to 16 columns in this 4-wave
// form, more in 32- or 48-column blocks of 2 key slots x 2 column halves
// (see decode_body).
// A sequence whose keys fit one split is finished by its workgroup. Otherwise
// each split stores its combined partial in the workspace and bumps the
// group's arrival counter; the last workgroup to arrive merges all partials
// (max, rescale, sum) and resets the counter to zero for the next call.
#include "duo_internal.h"
#include "mfma_common.h"
#include "qk_prologue.h"

#include <mutex>
#include <type_traits>

namespace duo {

constexpr int kDPitch = kD + 8;
constexpr int kTileElems = kDecodeKeys * kDPitch;  // one K or V tile in LDS

// One 32-key tile, global -> registers: rows ld_row + 4 j (clamped to the
// split's last slot), 16-byte chunk ld_chunk; each load instruction of the
// wave covers 4 consecutive 256-byte rows. The cache is read once per call,
// so the loads are non-temporal (they do not displace reused lines).
__device__ __forceinline__ void load_tile(const uint16_t* kbase, const uint16_t* vbase, int64_t k0,
                                          int64_t k_end, int ld_row, int ld_chunk, u32x4 (&stK)[8],
                                          u32x4 (&stV)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t slot = k0 + ld_row + 4 * j;
    slot = slot < k_end ? slot : k_end - 1;  // k_end >= 1 for a non-empty split
    stK[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + slot * kD + ld_chunk * 8));
    stV[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + slot * kD + ld_chunk * 8));
  }
}

// Block decode: key index k < n_valid is cache slot k, k >= n_valid is row
// k - n_valid of the block's own K/V (stride `bstride` elements per token).
// This wave loads rows ld_row + 4 j (j < kJ) of the tile starting at k0.
// kShared: another column block's workgroup streams the same keys at about
// the same time on this XCD, so the loads keep their lines in the L2 for it
// (ordinary loads; a single reader uses non-temporal ones). Verify blocks of
// 36-48 columns: 224 -> 207 us on the Duo decode workload's contexts.
template <int kJ, bool kShared>
__device__ __forceinline__ void load_tile_block(const uint16_t* kbase, const uint16_t* vbase,
                                                const uint16_t* kblk, const uint16_t* vblk, int64_t bstride,
                                                int64_t n_valid, int64_t k0, int64_t k_end, int ld_row,
                                                int ld_chunk, u32x4 (&stK)[kJ], u32x4 (&stV)[kJ]) {
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    int64_t key = k0 + ld_row + 4 * j;
    key = key < k_end ? key : k_end - 1;
    const bool cached = key < n_valid;
    const uint16_t* kp = cached ? kbase + key * kD : kblk + (key - n_valid) * bstride;
    const uint16_t* vp = cached ? vbase + key * kD : vblk + (key - n_valid) * bstride;
    const u32x4* ka = reinterpret_cast<const u32x4*>(kp + ld_chunk * 8);
    const u32x4* va = reinterpret_cast<const u32x4*>(vp + ld_chunk * 8);
    stK[j] = kShared ? *ka : __builtin_nontemporal_load(ka);
    stV[j] = kShared ? *va : __builtin_nontemporal_load(va);
  }
}

// Block decode visibility of key index k for this lane's query (column):
// position of cache slot k from the slot contract (a ring that has wrapped
// holds the newest positions below `past`), block key k at past + (k -
// n_valid); visible when not after the query and inside the class's band
// (sliding window of the main class, sink + recent of a streaming head).
struct BlockVis {
  int n_valid;     // cache slots
  int past;        // cached positions [0, past)
  int q_pos;       // this lane's query position
  int lo;          // lowest visible position of the band (INT32_MIN: none)
  int sink;        // positions below it are visible regardless of the band
  int ring_first;  // first ring slot, or -1 when slot = position
  int ring_len, wraps, rem;
  __device__ __forceinline__ int pos(int k) const {
    if (k >= n_valid) return past + (k - n_valid);
    if (ring_first < 0 || k < ring_first) return k;
    const int kr = k - ring_first;
    return ring_first + kr + ring_len * (wraps - (kr > rem ? 1 : 0));
  }
  __device__ __forceinline__ bool visible(int k) const {
    const int ps = pos(k);
    return ps <= q_pos && (ps < sink || ps >= lo);
  }
};

// Registers -> this wave's private LDS tile; the wave barrier orders the
// previous tile's reads before the overwrite and these writes before the reads.
__device__ __forceinline__ void stage_tile(uint16_t* sK, uint16_t* sV, int ld_row, int ld_chunk,
                                           const u32x4 (&stK)[8], const u32x4 (&stV)[8]) {
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int off = (ld_row + 4 * j) * kDPitch + ld_chunk * 8;
    *reinterpret_cast<u32x4*>(&sK[off]) = stK[j];
    *reinterpret_cast<u32x4*>(&sV[off]) = stV[j];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Block decode: this wave's rows ld_row + 4 j (j < 4, ld_row in [16 h,
// 16 h + 4)) into the key slot's shared tile; the workgroup barrier that
// follows orders them before the reads.
__device__ __forceinline__ void stage_rows(uint16_t* sK, uint16_t* sV, int ld_row, int ld_chunk,
                                           const u32x4 (&stK)[4], const u32x4 (&stV)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int off = (ld_row + 4 * j) * kDPitch + ld_chunk * 8;
    *reinterpret_cast<u32x4*>(&sK[off]) = stK[j];
    *reinterpret_cast<u32x4*>(&sV[off]) = stV[j];
  }
}

// One 32-key tile from LDS: S^T = K Q^T, mask slots >= k_end, online softmax
// update of (m, l, o) for the wave's 16 columns, O^T += V^T P^T.
// (kBlock: keys are masked per lane by `bv` on tiles where `mask_all` or the
// tile reaches the block keys or the item end.)
template <bool kBlock>
__device__ __forceinline__ void attend_tile(const uint16_t* sK, const uint16_t* sV, const bf16x8 (&qf)[4],
                                            int64_t k0, int64_t k_end, float c, int r16, int g, float& m,
                                            float& l, f32x4 (&o)[8], const BlockVis& bv, bool mask_all) {
  // At raised wave priority, so that a wave with a tile to attend gets the
  // issue slots before the SIMD's other wave, which is staging or waiting on
  // loads (verify blocks of 36-48 columns 4% faster).
  __builtin_amdgcn_s_setprio(1);
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[(16 * kt + r16) * kDPitch + 32 * ds + 8 * g]);
      s[kt] = mfma_16x16x32(a, qf[ds], s[kt]);
    }
  }
  if (kBlock) {
    if (mask_all || k0 + kDecodeKeys > bv.n_valid || k0 + kDecodeKeys > k_end) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t k = k0 + 16 * kt + 4 * g + i;
          if (k >= k_end || !bv.visible((int)k)) s[kt][i] = kNegInf;
        }
    }
  } else if (k0 + kDecodeKeys > k_end) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k0 + 16 * kt + 4 * g + i >= k_end) s[kt][i] = kNegInf;
  }
  float mx = s[0][0];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][i]);
  // lanes l, l ^ 16, l ^ 32, l ^ 48 hold the same column: row swaps on the
  // VALU (a shuffle is an LDS round trip, twice per tile on the attend path)
  mx = lane4_max(mx) * c;
  const bool up = mx > m + kRescaleThreshold;
  if (__any(up)) {
    const float a = up ? fast_exp2(m - mx) : 1.f;
    m = up ? mx : m;
    l *= a;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= a;
  }
  const float mu = (m == kNegInf) ? 0.f : m;
  float sum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = fast_exp2(__builtin_fmaf(s[kt][i], c, -mu));
      s[kt][i] = e;
      sum += e;
    }
  l += sum;
  const bf16x8 pb = pack_bf16(s[0], s[1]);
  const uint16_t* v0 = &sV[(4 * g + (r16 >> 2)) * kDPitch + 4 * (r16 & 3)];
  const uint16_t* v1 = v0 + 16 * kDPitch;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const bf16x8 a = cat_bf16(lds_read_tr16(v0 + 16 * dt), lds_read_tr16(v1 + 16 * dt));
    o[dt] = mfma_16x16x32(a, pb, o[dt]);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Output values (dim, dim + 1) of row bh: the unnormalised pair times the
// row's normaliser and, if the call has one, the output gate.
template <bool kFused>
__device__ __forceinline__ void write_out_pair(const DecodeParams& p, int64_t bh, int dim, float a0, float a1,
                                               float inv) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float f0 = inv, f1 = inv;
  if (kFused && p.gate != nullptr) {
    if (p.gate_mode == 2) {
      const float gf = gate_factor(bf16_bits_to_f32(p.gate[bh]));
      f0 *= gf;
      f1 *= gf;
    } else {
      const uint32_t gw = *reinterpret_cast<const uint32_t*>(p.gate + bh * kD + dim);
      f0 *= gate_factor(bf16_bits_to_f32(gw & 0xffffu));
      f1 *= gate_factor(bf16_bits_to_f32(gw >> 16));
    }
  }
  const bf16x2 r = __builtin_convertvector((f32x2{a0 * f0, a1 * f1}), bf16x2);
  *reinterpret_cast<bf16x2*>(p.out + bh * kD + dim) = r;
}

// One work item: (sequence, KV head, split) and, for the block decode, one
// block of 16 kNH of its (query token, query head) columns.
//
// kNH = 1 (the single-token decode, and a block of at most 16 columns): 4
// waves, each streaming its own 32-key tiles through a private LDS tile, two
// tiles in flight in registers.
// kNH = 2 (a block of 17-32 columns): 4 waves in 2 key slots x 2 column
// halves of 16. The two waves of a slot load half of each 32-key tile each (4
// half tiles in flight in registers) into the slot's shared LDS tile, and
// each attends it for its own 16 columns, so the cache is streamed once for
// 32 columns.
// kNH = 3 (blocks of 48 columns): the same 4 waves; half 0 attends column
// blocks 0 and 2, half 1 block 1, and the loads are split 6 : 10 row groups
// per tile so that both fit their registers with 3 tiles in flight. The
// cache is streamed once for 48 columns (verify blocks of 6-8 tokens at
// G = 6: T = 6 198 -> 175 us, T = 8 193 -> 182 us against two 32-column
// blocks on the Duo decode workload's contexts).
// Two workgroups of 4 waves share a CU in every form, so the split plan's
// items fill 512 resident slots (one 8-wave workgroup of 4 key slots per CU
// left this workload's 514 non-empty items a second, partly filled round:
// T = 4 / 6 / 8 147 / 172 / 179 -> 145 / 156 / 165 us).
// Out-of-contract lengths the decode kernels clamped (duo_device_errors),
// one word per device.
__device__ unsigned int g_decode_errors;

template <bool kBlock, int kNH, bool kFused, bool kShared = false>
__device__ __forceinline__ void decode_body(const DecodeParams& p) {
  static_assert(kNH == 1 || (kBlock && (kNH == 2 || kNH == 3)), "two or three column blocks only for the block decode");
  static_assert(!kShared || kNH >= 2, "shared key streams only between 32- or 48-column blocks");
  constexpr int kCols = 16 * kNH;
  constexpr int kHalves = kNH == 1 ? 1 : 2;
  // key slots per workgroup: 4 in the single-token form, 2 (x 2 halves) in
  // a block form
  constexpr int kSlots = kNH == 1 ? kDecodeWaves : 2;
  constexpr int kNW = kSlots * kHalves;  // waves per workgroup
  constexpr int kThreads = 64 * kNW;
  // K/V tiles (single token: one per wave; block: two per key slot, used
  // alternately); reused after the key loop for the combine/merge.
  __shared__ __attribute__((aligned(16))) uint16_t smem[kSlots * 2 * kHalves * kTileElems];
  static_assert(kSlots * kCols * kD * 4 <= (int)sizeof(smem), "combine area fits the tile area");
  static_assert(2 * 16 * kDecodeMaxSplits * 4 + 16 * 4 <= (int)sizeof(smem), "merge area fits the tile area");
  __shared__ float s_ml[kSlots][kCols][2];
  __shared__ int s_last;

  // Block decode: workgroup i runs on XCD i % 8 (round-robin dispatch); the
  // n_cb column blocks of one item are consecutive workgroups of the same
  // XCD, so the second and later readers of its K/V find them in that L2.
  int cb = 0, item = (int)blockIdx.x;
  if (kBlock) {
    const int x = (int)(blockIdx.x % kXcds), j = (int)(blockIdx.x / kXcds);
    cb = j % p.n_cb;
    item = (j / p.n_cb) * kXcds + x;
    if (item >= p.n_items) return;
  }
  const DecodeItem it = decode_item(p, item);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int slot = wave % kSlots;  // key slot: tiles k_begin + 32 (slot + kSlots t)
  const int half = wave / kSlots;  // column half (48 columns: half 0 takes blocks 0 and 2)
  const int lane = tid & 63;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int G = p.group;
  const int T = kBlock ? p.T : 1;

  const int64_t len = p.seq_lens[it.b];
  const int n_valid = (int)decode_valid_slots(p, it.cls, len > 0 ? len : 0);  // < 2^31
  const int n_keys = n_valid + (kBlock ? T : 0);
  const int n_planned = (it.cls == kStream) ? p.n_split_stream : p.n_split_main;
  const int n_needed = (n_keys + p.split_keys - 1) / p.split_keys;
  const int n_used = n_needed < n_planned ? n_needed : n_planned;  // a length beyond the planned maximum is cut
  if (tid == 0 && it.split == 0 && cb == 0) {
    // out-of-contract lengths, recorded once per (sequence, KV head)
    unsigned bad = 0u;
    if (it.cls != kStream && !p.main_ring && len > p.main_cap) bad |= kDevLengthPastCapacity;
    if (n_needed > n_planned) bad |= kDevLengthPastPlan;
    if (bad) atomicOr(&g_decode_errors, bad);
  }
  const int64_t k_begin = (int64_t)it.split * p.split_keys;
  int64_t k_end = k_begin + p.split_keys;
  if (k_end > n_keys) k_end = n_keys;

  // Columns of this item: (token t, head g) = (c / G, c % G), c in
  // [col0, col0 + n_cols); output row of column c.
  const int col0 = kCols * cb;
  const int n_cols = min(kCols, T * G - col0);
  const int n_half = (n_cols + 15) / 16;  // halves holding columns (uniform)
  auto row_of = [&](int c) -> int64_t {
    const int cc = col0 + c;
    return kBlock ? (((int64_t)it.b * T + cc / G) * p.hq + (int64_t)it.kvh * G + cc % G)
                  : ((int64_t)it.b * p.hq + (int64_t)it.kvh * G + cc);
  };
  auto head_of = [&](int c) -> int { return it.kvh * G + (kBlock ? (col0 + c) % G : col0 + c); };

  if (it.split >= n_used) {
    // empty split; split 0 of a sequence without keys writes the zero rows
    if (it.split == 0) {
      for (int e = tid; e < n_cols * (kD / 2); e += kThreads) {
        const int64_t row = row_of(e / (kD / 2));
        *reinterpret_cast<uint32_t*>(p.out + row * kD + 2 * (e % (kD / 2))) = 0u;
        if (p.lse != nullptr && (e % (kD / 2)) == 0)  // the sink alone, if any, forms the normaliser
          p.lse[row] = p.sink_logits != nullptr ? p.sink_logits[head_of(e / (kD / 2))] : kNegInf;
      }
    }
    return;
  }

  const uint16_t* kbase;
  const uint16_t* vbase;
  if (it.cls == kStream) {
    const int64_t off = ((int64_t)it.b * p.n_stream + it.rank) * (int64_t)(p.sink + p.recent) * kD;
    kbase = p.k_stream + off;
    vbase = p.v_stream + off;
  } else {
    const int64_t off = ((int64_t)it.b * p.n_main + it.rank) * p.main_cap * kD;
    kbase = p.k_main + off;
    vbase = p.v_main + off;
  }

  // Q fragments of this wave's half: lane column hc = 16 half + r16 (zero
  // beyond the item's columns).
  const int hc = 16 * half + r16;
  bf16x8 qf[4];
  {
    const bool ok = hc < n_cols;
    const uint16_t* src = p.q + row_of(ok ? hc : 0) * kD + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ds) : u32x4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8, raw);
    }
    // RMSNorm + RoPE of q: the single-token query sits at len - 1, block
    // token t at past + t.
    if (kFused && p.qpro_on) prologue_frag(qf, kBlock ? (int)len + (col0 + hc) / G : (int)len - 1, g, p.qpro);
  }
  // 48-column blocks: half 0 also attends column block 2 (lane column hc2)
  const int hc2 = 32 + r16;
  // Block decode: visibility of each key for this lane's query token.
  BlockVis bv{};
  bool mask_all = false;
  const uint16_t* kblk = nullptr;
  const uint16_t* vblk = nullptr;
  const int64_t bstride = (int64_t)p.hkv * kD;
  if (kBlock) {
    const int past = len > 0 ? (int)len : 0;  // cached positions [0, past)
    const int t = (hc < n_cols ? col0 + hc : col0) / G;
    bv.n_valid = n_valid;
    bv.past = past;
    bv.q_pos = past + t;
    bv.lo = INT32_MIN;
    bv.sink = 0;
    bv.ring_first = -1;
    int ring_len = 0, first = 0;
    if (it.cls == kStream) {
      bv.lo = bv.q_pos - p.recent + 1;
      bv.sink = p.sink;
      first = p.sink;
      ring_len = p.recent;
    } else if (p.main_ring) {
      bv.lo = bv.q_pos - p.window + 1;
      ring_len = (int)p.main_cap;
    }
    if (ring_len > 0 && past > first + ring_len) {  // the ring has wrapped
      const int rel = past - 1 - first;
      bv.ring_first = first;
      bv.ring_len = ring_len;
      bv.wraps = rel / ring_len;
      bv.rem = rel - bv.wraps * ring_len;
    }
    mask_all = ring_len > 0;  // a band: the oldest cached positions can fall out of it

    kblk = p.k_new + ((int64_t)it.b * T * p.hkv + it.kvh) * kD;
    vblk = p.v_new + ((int64_t)it.b * T * p.hkv + it.kvh) * kD;
  }

  const float c = p.scale_log2;
  float m = kNegInf, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Tiles of key slot `slot` start at k_begin + 32 * (slot + kSlots t). Loads are
  // issued unconditionally so the wait counts stay exact: a tile past the
  // split end reads the last valid key and is fully masked, leaving (m, l, o)
  // unchanged.
  const int64_t stride = (int64_t)kDecodeKeys * kSlots;
  const int64_t first = k_begin + (int64_t)kDecodeKeys * slot;
  const int ld_chunk = lane & 15;
  if (kNH == 1) {
    uint16_t* sK = smem + wave * 2 * kTileElems;
    uint16_t* sV = sK + kTileElems;
    const int ld_row = lane >> 4;
    const int64_t nt = first < k_end ? (k_end - first + stride - 1) / stride : 0;
    // Two tiles in flight (register buffers A and B, used alternately).
    // (scheduling barriers keep each tile's 16 loads contiguous in issue
    // order, so waiting for one buffer never waits for the other)
    auto load = [&](int64_t k0, u32x4 (&bk)[8], u32x4 (&bvv)[8]) {
      if (kBlock)
        load_tile_block<8, false>(kbase, vbase, kblk, vblk, bstride, n_valid, k0, k_end, ld_row, ld_chunk, bk, bvv);
      else
        load_tile(kbase, vbase, k0, k_end, ld_row, ld_chunk, bk, bvv);
    };
    u32x4 aK[8], aV[8], bK[8], bV[8];
    load(first, aK, aV);
    __builtin_amdgcn_sched_barrier(0);
    load(first + stride, bK, bV);
    __builtin_amdgcn_sched_barrier(0);
    int64_t t = 0;
    for (; t + 2 < nt; t += 2) {
      const int64_t k0 = first + t * stride;
      stage_tile(sK, sV, ld_row, ld_chunk, aK, aV);
      __builtin_amdgcn_sched_barrier(0);
      load(k0 + 2 * stride, aK, aV);
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kBlock>(sK, sV, qf, k0, k_end, c, r16, g, m, l, o, bv, mask_all);
      __builtin_amdgcn_sched_barrier(0);
      stage_tile(sK, sV, ld_row, ld_chunk, bK, bV);
      __builtin_amdgcn_sched_barrier(0);
      load(k0 + 3 * stride, bK, bV);
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kBlock>(sK, sV, qf, k0 + stride, k_end, c, r16, g, m, l, o, bv, mask_all);
      __builtin_amdgcn_sched_barrier(0);
    }
    // The last pass (the wave's last one or two tiles) issues no loads: a
    // batch-64 sliding-window decode streams 4 tiles per wave, and the two
    // extra tile loads of the clamped last key per wave cost 4% there
    // (27.3 -> 26.2 us). Peeled rather than predicated: a predicated load
    // makes the compiler wait for every outstanding load before staging.
    if (t < nt) {
      const int64_t k0 = first + t * stride;
      stage_tile(sK, sV, ld_row, ld_chunk, aK, aV);
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kBlock>(sK, sV, qf, k0, k_end, c, r16, g, m, l, o, bv, mask_all);
      __builtin_amdgcn_sched_barrier(0);
      stage_tile(sK, sV, ld_row, ld_chunk, bK, bV);
      __builtin_amdgcn_sched_barrier(0);
      attend_tile<kBlock>(sK, sV, qf, k0 + stride, k_end, c, r16, g, m, l, o, bv, mask_all);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (kNH == 2) {
    // The slot's two LDS tiles, used alternately: one workgroup barrier per
    // tile orders this tile's staging before its reads, and every read of
    // the other tile (two tiles back) before its next staging.
    uint16_t* sK0 = smem + slot * 4 * kTileElems;
    uint16_t* sV0 = sK0 + kTileElems;
    uint16_t* sK1 = sV0 + kTileElems;
    uint16_t* sV1 = sK1 + kTileElems;
    const int ld_row = 16 * half + (lane >> 4);  // rows ld_row + 4 j, j < 4
    // the same trip count in every wave (barriers): slot 0 has the most tiles
    const int64_t nt = (k_end - k_begin + stride - 1) / stride;
    u32x4 xK[4][4], xV[4][4];  // four half tiles in flight
    auto load = [&](int64_t k0, u32x4 (&bk)[4], u32x4 (&bvv)[4]) {
      load_tile_block<4, kShared>(kbase, vbase, kblk, vblk, bstride, n_valid, k0, k_end, ld_row, ld_chunk, bk, bvv);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load(first + i * stride, xK[i], xV[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    auto step = [&](int64_t t, auto with_load, u32x4 (&bk)[4], u32x4 (&bvv)[4], uint16_t* sK, uint16_t* sV) {
      const int64_t k0 = first + t * stride;
      stage_rows(sK, sV, ld_row, ld_chunk, bk, bvv);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(with_load)::value) load(k0 + 4 * stride, bk, bvv);
      __builtin_amdgcn_sched_barrier(0);
      if (half < n_half)  // a half without columns only helps load and stage
        attend_tile<kBlock>(sK, sV, qf, k0, k_end, c, r16, g, m, l, o, bv, mask_all);
      __builtin_amdgcn_sched_barrier(0);
    };
    // Whole passes of four steps, then at most three steps that load
    // nothing. (A pass that could break out after any step left the loop
    // head with an inexact wait: its first staging waited for all four half
    // tiles in flight, draining the stream every fourth tile; verify blocks
    // of 6-8 tokens 204 -> 194 us on the Duo decode workload's contexts.)
    const std::true_type loads{};
    const std::false_type no_loads{};
    int64_t t = 0;
    for (; t + 4 <= nt; t += 4) {
      step(t, loads, xK[0], xV[0], sK0, sV0);
      step(t + 1, loads, xK[1], xV[1], sK1, sV1);
      step(t + 2, loads, xK[2], xV[2], sK0, sV0);
      step(t + 3, loads, xK[3], xV[3], sK1, sV1);
    }
    if (t < nt) step(t, no_loads, xK[0], xV[0], sK0, sV0);
    if (t + 1 < nt) step(t + 1, no_loads, xK[1], xV[1], sK1, sV1);
    if (t + 2 < nt) step(t + 2, no_loads, xK[2], xV[2], sK0, sV0);
  } else {
    // 48 columns, the cache streamed once: a 32-key tile is 16 groups of 4
    // rows (8 of K, 8 of V); the waves of half 0, which attend two column
    // blocks, load 6 groups of each tile, those of half 1 the other 10, so
    // that both fit their registers with three tiles in flight (three
    // quarters of the 32-column form's bytes in flight per CU; four tiles
    // spilled 72 registers).
    uint16_t* sK0 = smem + slot * 4 * kTileElems;
    uint16_t* sV0 = sK0 + kTileElems;
    uint16_t* sK1 = sV0 + kTileElems;
    uint16_t* sV1 = sK1 + kTileElems;
    const int64_t nt = (k_end - k_begin + stride - 1) / stride;
    // state of column block 2 (half 0 only)
    struct Second {
      bf16x8 qf[4];
      BlockVis bv;
      float m, l;
      f32x4 o[8];
    };
    auto stream = [&](auto n_groups, auto group0, auto two_blocks, Second& sec) {
      constexpr int kG = decltype(n_groups)::value;
      constexpr int kG0 = decltype(group0)::value;
      constexpr bool kTwo = decltype(two_blocks)::value;
      constexpr int kDepth = 3;  // tiles in flight
      u32x4 x[kDepth][kG];
      auto load = [&](int64_t k0, u32x4 (&bx)[kG]) {
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          const int gi = kG0 + i;
          int64_t key = k0 + 4 * (gi & 7) + (lane >> 4);
          key = key < k_end ? key : k_end - 1;
          const bool cached = key < n_valid;
          const uint16_t* src = gi < 8 ? (cached ? kbase + key * kD : kblk + (key - n_valid) * bstride)
                                       : (cached ? vbase + key * kD : vblk + (key - n_valid) * bstride);
          const u32x4* a = reinterpret_cast<const u32x4*>(src + ld_chunk * 8);
          bx[i] = kShared ? *a : __builtin_nontemporal_load(a);
        }
      };
#pragma unroll
      for (int i = 0; i < kDepth; ++i) {
        load(first + i * stride, x[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      auto step = [&](int64_t t, auto with_load, u32x4 (&bx)[kG], uint16_t* sK, uint16_t* sV) {
        const int64_t k0 = first + t * stride;
#pragma unroll
        for (int i = 0; i < kG; ++i) {
          const int gi = kG0 + i;
          const int off = (4 * (gi & 7) + (lane >> 4)) * kDPitch + ld_chunk * 8;
          *reinterpret_cast<u32x4*>(&(gi < 8 ? sK : sV)[off]) = bx[i];
        }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(with_load)::value) load(k0 + kDepth * stride, bx);
        __builtin_amdgcn_sched_barrier(0);
        if (half < n_half) attend_tile<kBlock>(sK, sV, qf, k0, k_end, c, r16, g, m, l, o, bv, mask_all);
        if constexpr (kTwo)
          if (n_half > 2) attend_tile<kBlock>(sK, sV, sec.qf, k0, k_end, c, r16, g, sec.m, sec.l, sec.o, sec.bv, mask_all);
        __builtin_amdgcn_sched_barrier(0);
      };
      const std::true_type loads{};
      const std::false_type no_loads{};
      // passes of six steps (register buffer t mod 3, LDS tile t mod 2);
      // then at most five steps, of which only the first three load (their
      // tiles may lie past the end: clamped reads, fully masked)
      int64_t t = 0;
      for (; t + 6 <= nt; t += 6) {
        step(t, loads, x[0], sK0, sV0);
        step(t + 1, loads, x[1], sK1, sV1);
        step(t + 2, loads, x[2], sK0, sV0);
        step(t + 3, loads, x[0], sK1, sV1);
        step(t + 4, loads, x[1], sK0, sV0);
        step(t + 5, loads, x[2], sK1, sV1);
      }
      if (t < nt) step(t, loads, x[0], sK0, sV0);
      if (t + 1 < nt) step(t + 1, loads, x[1], sK1, sV1);
      if (t + 2 < nt) step(t + 2, loads, x[2], sK0, sV0);
      if (t + 3 < nt) step(t + 3, no_loads, x[0], sK1, sV1);
      if (t + 4 < nt) step(t + 4, no_loads, x[1], sK0, sV0);
    };
    if (half == 0) {
      Second sec;
      {
        const bool ok = hc2 < n_cols;
        const uint16_t* src = p.q + row_of(ok ? hc2 : 0) * kD + 8 * g;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ds) : u32x4{0u, 0u, 0u, 0u};
          sec.qf[ds] = __builtin_bit_cast(bf16x8, raw);
        }
        if (kFused && p.qpro_on) prologue_frag(sec.qf, (int)len + (col0 + hc2) / G, g, p.qpro);
        // the same bands, for the query token of lane column hc2
        sec.bv = bv;
        sec.bv.q_pos = bv.past + (ok ? col0 + hc2 : col0) / G;
        if (bv.lo != INT32_MIN) sec.bv.lo = bv.lo + (sec.bv.q_pos - bv.q_pos);
        sec.m = kNegInf;
        sec.l = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) sec.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      stream(std::integral_constant<int, 6>{}, std::integral_constant<int, 0>{}, std::true_type{}, sec);
      sec.l = lane4_sum(sec.l);
      // every wave is past its last tile: block 2's partial into the
      // combine area (over the tiles)
      __syncthreads();
      float* comb = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<f32x4*>(&comb[(slot * kCols + hc2) * kD + 16 * dt + 4 * g]) = sec.o[dt];
      if (g == 0) {
        s_ml[slot][hc2][0] = sec.m;
        s_ml[slot][hc2][1] = sec.l;
      }
    } else {
      Second none;
      stream(std::integral_constant<int, 10>{}, std::integral_constant<int, 6>{}, std::false_type{}, none);
      __syncthreads();
    }
  }
  l = lane4_sum(l);

  // ---- combine the key slots: acc[slot][col][dim] in LDS (reuses the tile area)
  __syncthreads();
  float* comb = reinterpret_cast<float*>(smem);  // [4][kCols][128] floats
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *reinterpret_cast<f32x4*>(&comb[(slot * kCols + hc) * kD + 16 * dt + 4 * g]) = o[dt];
  if (g == 0) {
    s_ml[slot][hc][0] = m;
    s_ml[slot][hc][1] = l;
  }

  __syncthreads();

  // thread -> (column, dim pair) of the item's columns; 64 threads per column
  const bool single = (n_used == 1);
  for (int e = tid; e < n_cols * (kD / 2); e += kThreads) {
    const int col = e / (kD / 2);
    const int dim = 2 * (e % (kD / 2));
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kSlots; ++w) M = fmaxf(M, s_ml[w][col][0]);
    float L = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int w = 0; w < kSlots; ++w) {
      const float mw = s_ml[w][col][0];
      const float sc = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      L += sc * s_ml[w][col][1];
      a0 += sc * comb[(w * kCols + col) * kD + dim];
      a1 += sc * comb[(w * kCols + col) * kD + dim + 1];
    }
    const int64_t row = row_of(col);
    if (single) {
      const RowNorm rn = row_norm(M, L, kFused ? p.sink_logits : nullptr, head_of(col));
      write_out_pair<kFused>(p, row, dim, a0, a1, rn.inv);
      if (p.lse != nullptr && dim == 0) p.lse[row] = rn.lse;
    } else {
      const int64_t wslot = row * p.n_split_max + it.split;
      coherent_store(p.ws_acc + wslot * kD + dim, a0);
      coherent_store(p.ws_acc + wslot * kD + dim + 1, a1);
      if (dim == 0) {
        coherent_store(p.ws_ml + wslot * 2 + 0, M);
        coherent_store(p.ws_ml + wslot * 2 + 1, L);
      }
    }
  }
  if (single) return;

  // ---- split-K: publish this partial; the last workgroup of the group merges.
  // Partials travel through device-coherent (sc1) stores and loads, which
  // bypass the per-XCD L2 caches; each wave drains its stores before the
  // arrival counter is bumped, so no cache-wide writeback fence is needed.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* counter = p.ws_count + ((int64_t)it.b * p.hkv + it.kvh) * p.n_cb + cb;
  if (tid == 0)
    s_last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_used - 1);
  __syncthreads();
  if (!s_last) return;

  // Merge, 16 columns at a time: (max, sum) of every (column, split) into
  // LDS with all loads in flight, then per-column max / weights / normaliser,
  // then the weighted sum of the partial outputs. The merge runs in the
  // launch's tail (the other workgroups have finished), so its load latency
  // is paid in full: each thread owns 4 dims of one column and keeps 8
  // splits of loads in flight, with no cross-wave reduction.
  float* s_m = reinterpret_cast<float*>(smem);  // [16][kDecodeMaxSplits]
  float* s_w = s_m + 16 * kDecodeMaxSplits;       // [16][kDecodeMaxSplits] weights
  float* s_L = s_w + 16 * kDecodeMaxSplits;       // [16] output factors (1 / normaliser)
  for (int hb = 0; hb < n_half; ++hb) {
    const int c0 = 16 * hb;                       // first column of this half
    const int nc = min(16, n_cols - c0);
    if (hb > 0) __syncthreads();                  // the previous half is done with the LDS
    for (int e = tid; e < nc * n_used; e += kThreads) {
      const int h = e / n_used, sp = e % n_used;
      const float* ml = p.ws_ml + (row_of(c0 + h) * p.n_split_max + sp) * 2;
      s_m[h * kDecodeMaxSplits + sp] = coherent_load(ml);
      s_w[h * kDecodeMaxSplits + sp] = coherent_load(ml + 1);
    }
    __syncthreads();
    for (int h = wave; h < nc; h += kNW) {
      float M = kNegInf;
      for (int sp = lane; sp < n_used; sp += 64) M = fmaxf(M, s_m[h * kDecodeMaxSplits + sp]);
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
      float L = 0.f;
      for (int sp = lane; sp < n_used; sp += 64) {
        const float ms = s_m[h * kDecodeMaxSplits + sp];
        const float w = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
        L += w * s_w[h * kDecodeMaxSplits + sp];
        s_w[h * kDecodeMaxSplits + sp] = w;
      }
#pragma unroll
      for (int x = 32; x >= 1; x >>= 1) L += __shfl_xor(L, x);
      if (lane == 0) {
        const RowNorm rn = row_norm(M, L, kFused ? p.sink_logits : nullptr, head_of(c0 + h));
        s_L[h] = rn.inv;
        if (p.lse != nullptr) p.lse[row_of(c0 + h)] = rn.lse;
      }
    }
    __syncthreads();
    // weighted sum of the partial outputs: thread -> (column h, dims d..d+3),
    // 32 threads per column, walking every split with kMergeU splits of
    // 8-byte coherent loads in flight (past the last split the loads repeat
    // it with weight 0, so they need no predicate)
    constexpr int kMergeU = 8;
    for (int e = tid; e < nc * 32; e += kThreads) {
      const int h = e >> 5;
      const int d = 4 * (e & 31);
      const int64_t row = row_of(c0 + h);
      const float* src = p.ws_acc + row * p.n_split_max * kD + d;
      const float* wts = s_w + h * kDecodeMaxSplits;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int sp0 = 0; sp0 < n_used; sp0 += kMergeU) {
        f32x2 lo[kMergeU], hi[kMergeU];
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
          const float* q = src + (int64_t)min(sp0 + u, n_used - 1) * kD;
          lo[u] = coherent_load2(q);
          hi[u] = coherent_load2(q + 2);
        }
#pragma unroll
        for (int u = 0; u < kMergeU; ++u) {
          const float w = sp0 + u < n_used ? wts[sp0 + u] : 0.f;
          a0 += w * lo[u].x;
          a1 += w * lo[u].y;
          a2 += w * hi[u].x;
          a3 += w * hi[u].y;
        }
      }
      write_out_pair<kFused>(p, row, d, a0, a1, s_L[h]);
      write_out_pair<kFused>(p, row, d + 2, a2, a3, s_L[h]);
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // next call
}

// Plain kernels carry no prologue or epilogue code (it measurably slows the
// plain path even when skipped); the fused ones are used when a call passes
// a q prologue, sink logits or a gate.
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) { decode_body<false, 1, false>(p); }
__global__ __launch_bounds__(256, 2) void decode_block16_kernel(DecodeParams p) { decode_body<true, 1, false>(p); }
__global__ __launch_bounds__(256, 2) void decode_block_kernel(DecodeParams p) { decode_body<true, 2, false>(p); }
__global__ __launch_bounds__(256, 2) void decode_block48_kernel(DecodeParams p) { decode_body<true, 3, false>(p); }
__global__ __launch_bounds__(256, 2) void decode_block48_shared_kernel(DecodeParams p) {
  decode_body<true, 3, false, true>(p);
}
__global__ __launch_bounds__(256, 2) void decode_block_shared_kernel(DecodeParams p) {
  decode_body<true, 2, false, true>(p);
}
__global__ __launch_bounds__(256, 2) void decode_fused_kernel(DecodeParams p) { decode_body<false, 1, true>(p); }
__global__ __launch_bounds__(256, 2) void decode_block16_fused_kernel(DecodeParams p) { decode_body<true, 1, true>(p); }
__global__ __launch_bounds__(256, 2) void decode_block_fused_kernel(DecodeParams p) { decode_body<true, 2, true>(p); }
__global__ __launch_bounds__(256, 2) void decode_block48_fused_kernel(DecodeParams p) { decode_body<true, 3, true>(p); }
__global__ __launch_bounds__(256, 2) void decode_block48_shared_fused_kernel(DecodeParams p) {
  decode_body<true, 3, true, true>(p);
}
__global__ __launch_bounds__(256, 2) void decode_block_shared_fused_kernel(DecodeParams p) {
  decode_body<true, 2, true, true>(p);
}

static bool fused(const DecodeParams& p) { return p.qpro_on || p.sink_logits != nullptr || p.gate != nullptr; }

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.n_items > 0)
    hipLaunchKernelGGL(fused(p) ? decode_fused_kernel : decode_kernel, dim3((unsigned)p.n_items), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_block(const DecodeParams& p, hipStream_t s) {
  const int64_t items8 = ((int64_t)p.n_items + kXcds - 1) / kXcds * kXcds;
  if (p.n_items > 0) {
    const dim3 grid((unsigned)(items8 * p.n_cb));
    const bool f = fused(p);
    const int cols = p.T * p.group;
    if (cols <= 16)  // one 16-column block: the 4-wave form
      hipLaunchKernelGGL(f ? decode_block16_fused_kernel : decode_block16_kernel, grid, dim3(256), 0, s, p);
    else if (cols <= 32)  // one 32-column block
      hipLaunchKernelGGL(f ? decode_block_fused_kernel : decode_block_kernel, grid, dim3(256), 0, s, p);
    else if (p.n_cb == 1)  // one 48-column block
      hipLaunchKernelGGL(f ? decode_block48_fused_kernel : decode_block48_kernel, grid, dim3(256), 0, s, p);
    else  // several 48-column blocks stream the same keys
      hipLaunchKernelGGL(f ? decode_block48_shared_fused_kernel : decode_block48_shared_kernel, grid, dim3(256), 0,
                         s, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- no-allocation decode
// Scratch held by the library for duo_attn_decode_noalloc (callers that cannot
// allocate device memory): the same layout as a caller's decode workspace, in
// one file-scope device array per GPU, kept until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address is resolved once per device with hipGetSymbolAddress, with
// that device current, and only that address is handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t decode_device_errors(uint32_t* bits, bool clear) {
  unsigned v = 0u;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_decode_errors), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear && v != 0u) {
    const unsigned z = 0u;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_decode_errors), &z, sizeof z, 0, hipMemcpyHostToDevice);
  }
  *bits |= v;
  return e;
}

hipError_t launch_fill_zero(int32_t* p, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace duo
