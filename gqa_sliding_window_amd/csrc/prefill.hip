// Prefill attention kernel (gfx950): flash-style online softmax, QK^T and PV
// on bf16 MFMA with fp32 accumulation, K/V tiles staged in LDS, masked tiles
// skipped per head class.
//
// What is computed (per query row i of head h, KV head h / G): softmax over
// the visible key positions of scale * q.k, applied to v. Visibility per head
// class: full-context heads see the causal prefix (or the causal window of a
// sliding layer); streaming heads see sink positions plus the `recent`
// positions ending at i (model card "DuoAttention Laguna Adapter", "Summary"
// and "Why It Works"; Laguna-M.1-8bit blog post, sliding-window and
// mask-generation sections).
//
// Workgroup = 4 waves of 32 query rows (two 16-row MFMA column blocks each):
// 64 rows of two query heads of one KV head, or 128 rows of one query head
// when the group size is odd. Keys come in 64-key tiles over at
// most two ranges (causal prefix / window band, or sink + recent band); tiles
// outside the ranges are never visited and only tiles on a range edge, the
// diagonal or a band edge evaluate the per-element predicate. Keys before
// start_pos are read from the cache (slot per class), the chunk's own keys
// from the k/v inputs. Positions are 32-bit (the host keeps them 1024 below
// 2^31, so tile and row bounds formed past the last position cannot
// overflow); a tile that lies wholly in the chunk or in a contiguous stretch
// of the cache is addressed from one base pointer, other tiles row by row.
#include "duo_internal.h"
#include "mfma_common.h"
#include "qk_prologue.h"

namespace duo {

// LDS tiles are unpadded (256-byte rows) with their 16-byte chunks
// XOR-swizzled by row: logical chunk c of row r sits at chunk c ^ (r & 15) of
// a K row and c ^ 2 (r & 7) of a V row. A K fragment read (16 rows x one
// chunk per 16 lanes) and a V transpose read (8 rows x 32 bytes per 32
// lanes) then touch distinct banks, and one load instruction fills 4 whole
// rows with its lanes in aligned 64-byte groups.
constexpr int kPitch = kD;   // K and V rows: 256 bytes
constexpr int kVPitch = kD;
constexpr int kNegBig = -0x7fffffff;
// Query rows per wave, in 16-row MFMA column blocks: 32 rows per wave. (64
// rows per wave would halve the LDS operand reads per MFMA, but its
// accumulators and Q fragments do not fit one wave's registers without spills.)
constexpr int kRT = 2;
constexpr int kWaves = kPrefillWaves;  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
static_assert(kPrefillWaveRows == 16 * kRT, "32 rows per wave");

struct TileRange {
  int lo, hi;      // visible key positions of the range (inclusive)
  int span;        // > 0: causal band of this width ending at the query
  int first;       // first tile start (lo rounded down to 64)
};

// A wave's per-tile tests on a key range, as intervals of the tile start lo
// (keys lo .. lo + 63), formed once per work item: the tile is visible to
// the wave's rows [qw0, qw1] when vlo <= lo <= vhi, and every key of it is
// visible to every one of those rows when mlo <= lo <= mhi.
struct TileTest {
  int vlo, vhi, mlo, mhi;
};

__device__ __forceinline__ TileTest tile_test(const TileRange& r, int qw0, int qw1, bool wave_active) {
  constexpr int64_t kLow = kNegBig;
  TileTest t;
  // some key lo .. lo + 63 in the band of row qw0: lo + 63 >= qw0 - span + 1;
  // some key not after row qw1: lo <= qw1
  t.vlo = r.span > 0 ? (int)max((int64_t)qw0 - r.span - (kPrefillKeys - 2), kLow) : kNegBig;
  t.vhi = wave_active ? qw1 : kNegBig;
  // lo >= r.lo, lo + 63 <= min(r.hi, qw0), lo >= qw1 - span + 1
  t.mlo = r.span > 0 ? (int)max((int64_t)r.lo, (int64_t)qw1 - r.span + 1) : r.lo;
  t.mhi = min(r.hi, qw0) - (kPrefillKeys - 1);
  return t;
}

struct Src {
  const uint16_t* k;
  const uint16_t* v;
};

// Everything the loader needs about one (sequence, KV head).
struct KvSrc {
  const uint16_t* ck;    // chunk K/V at position P, this (b, kvh)
  const uint16_t* cv;
  int64_t cstride;       // elements between consecutive chunk positions
  const uint16_t* mk;    // cache rows of this (b, class, rank), slot 0
  const uint16_t* mv;
  int P;                 // start_pos
  int cls;
  int ring_cap;          // main ring capacity (0 = contiguous main cache)
  int sink, recent;
  int chunk_end;          // P + T: first position past the chunk
};

// Cache slot of a past position (library slot contract, see duo_attn.h).
__device__ __forceinline__ int cache_slot(const KvSrc& s, int pos) {
  if (s.cls == kStream) return pos < s.sink ? pos : s.sink + (pos - s.sink) % s.recent;
  return s.ring_cap ? pos % s.ring_cap : pos;
}

__device__ __forceinline__ Src row_src(const KvSrc& s, int pos) {
  Src r;
  if (pos >= s.P) {
    const int64_t off = (int64_t)(pos - s.P) * s.cstride;
    r.k = s.ck + off;
    r.v = s.cv + off;
  } else {
    const int64_t off = (int64_t)cache_slot(s, pos) * kD;
    r.k = s.mk + off;
    r.v = s.mv + off;
  }
  return r;
}

// Addressing of one tile's rows. A tile that starts in the chunk, or lies
// wholly in a stretch of the cache where slot = position, is loaded from one
// base pointer and a row stride, whatever part of it the key range covers:
// its rows outside the range are valid keys and values whose logits are
// masked, and rows past the chunk's end lie outside the load's buffer and
// read as zeros. Other tiles are loaded row by row (positions outside the
// range clamped onto it: their logits are masked, their values are finite
// data).
struct TileAddr {
  const uint16_t* k;
  const uint16_t* v;
  uint32_t stride_b;  // bytes between consecutive rows (fast form)
  uint32_t bytes;     // bytes of the tile's rows that exist, from k / v (fast form)
  bool general;       // row-by-row form
};

__device__ __forceinline__ TileAddr tile_addr(const KvSrc& s, int lo) {
  const int hi = lo + kPrefillKeys - 1;
  TileAddr a;
  a.general = false;
  if (lo >= s.P) {
    const int64_t off = (int64_t)(lo - s.P) * s.cstride;
    a.k = s.ck + off;
    a.v = s.cv + off;
    a.stride_b = (uint32_t)s.cstride * 2u;
    a.bytes = (uint32_t)min(s.chunk_end - 1 - lo, kPrefillKeys - 1) * a.stride_b + kD * 2u;
    return a;
  }
  const bool contiguous_cache = hi < s.P && (s.cls == kStream ? hi < s.sink : s.ring_cap == 0);
  if (contiguous_cache) {
    const int64_t off = (int64_t)lo * kD;
    a.k = s.mk + off;
    a.v = s.mv + off;
    a.stride_b = kD * 2u;
    a.bytes = kPrefillKeys * kD * 2u;
    return a;
  }
  a.k = s.mk;
  a.v = s.mv;
  a.stride_b = 0;
  a.bytes = 0;
  a.general = true;
  return a;
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS loads of a K (kV = false) or V tile: 16 instructions
// of 64 lanes x 16 bytes, instruction J filling rows 4 J .. 4 J + 3, dealt
// round-robin to the waves (wave w takes J = w + 4 jj). Lane l of instruction
// J fetches row 4 J + l / 16 at the logical chunk that the row's swizzle
// puts in physical chunk l % 16; row & 15 (and row & 7) is the same for all
// of a wave's instructions, so each lane's chunk is fixed.
struct DmaLane {
  uint32_t row;      // lane / 16: row within the instruction's 4
  uint32_t kchunkb;  // byte offset of the K chunk this lane fetches
  uint32_t vchunkb;  // byte offset of the V chunk this lane fetches
  __device__ __forceinline__ void init(int wave, int lane) {
    row = (uint32_t)(lane >> 4);
    const uint32_t r = 4u * (uint32_t)wave + row;  // tile row mod 16 of every instruction of this wave
    kchunkb = (((uint32_t)lane & 15u) ^ (r & 15u)) * 16u;
    vchunkb = (((uint32_t)lane & 15u) ^ (2u * (r & 7u))) * 16u;
  }
};
constexpr int kDmaPerWave = kPrefillKeys / 4 / kWaves;  // 4 instructions per wave and tile array
static_assert(kPrefillKeys % (4 * kWaves) == 0, "tile must be whole load instructions per wave");

template <bool kV>
__device__ __forceinline__ void dma_tile(uint16_t* lds, const KvSrc& s, const TileRange& r, int lo,
                                         const TileAddr& ta, int wave, const DmaLane& dl) {
  const uint32_t chunkb = kV ? dl.vchunkb : dl.kchunkb;
  if (!ta.general) {
    // buffer loads from a raw buffer over the tile's rows (descriptor word
    // 3: 32-bit data format) + a 32-bit lane offset (row < 64, stride < 2^24
    // bytes). A global load into LDS is a flat access to both memories, and
    // while one is in flight the compiler makes every LDS read wait for all
    // outstanding LDS operations; with buffer loads in flight the K and V
    // fragment reads keep their partial waits.
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(kV ? ta.v : ta.k), 0, (int)ta.bytes, 0x00020000);
    const uint32_t lane_off = __umul24(dl.row, ta.stride_b) + chunkb;
#pragma unroll
    for (int jj = 0; jj < kDmaPerWave; ++jj) {
      const int J = wave + kWaves * jj;
      const uint32_t off = lane_off + (uint32_t)(4 * J) * ta.stride_b;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + J * 512), 16, off, 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int jj = 0; jj < kDmaPerWave; ++jj) {
    const int J = wave + kWaves * jj;
    int pos = lo + 4 * J + (int)dl.row;
    pos = pos < r.lo ? r.lo : (pos > r.hi ? r.hi : pos);
    const Src rs = row_src(s, pos);
    const char* src = reinterpret_cast<const char*>(kV ? rs.v : rs.k) + chunkb;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds + J * 512), 16, 0, 0);
  }
  // the row-by-row form (tiles across start_pos or in a cache ring) waits
  // for its global loads here, so that none is in flight at the LDS reads
  __builtin_amdgcn_s_waitcnt(0);
}

// kHeads query heads of one KV head per workgroup: waves w and w + 2 of a
// two-head workgroup take the same 32 rows of the two heads, so every wave
// sees the same key band and a tile visible to one is visible to all (a
// sliding-window layer walks 9 tiles per workgroup instead of 10 for 128
// rows of one head: 6% faster there, 10% on a 1 x 1024 layer).
template <bool kFused, int kHeads>
__device__ __forceinline__ void prefill_body(const PrefillParams& p) {
  constexpr int kRowWaves = kWaves / kHeads;
  constexpr int kRows = kRowWaves * kPrefillWaveRows;
  // Two K/V buffers as separate arrays, so that loads into one are known not
  // to alias reads of the other.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[kPrefillKeys * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[kPrefillKeys * kVPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[kPrefillKeys * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[kPrefillKeys * kVPitch];

  __shared__ int s_last;
  __shared__ int s_fin[8];  // work item fields for the finish (b, qhead, qa, qb, pieces used, unit, piece)
  const PrefillItem it = prefill_item(p, blockIdx.x);
  if (!it.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rwave = wave % kRowWaves;
  const int qhead = it.qhead + wave / kRowWaves;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int P = (int)p.start_pos;
  const int last = P + p.T - 1;
  const int qa = P + it.qtile * kRows;
  const int qb = min(qa + kRows - 1, last);
  const int qw0 = qa + rwave * 16 * kRT;
  const int qw1 = min(qw0 + 16 * kRT - 1, qb);
  const bool wave_active = qw0 <= qb;

  // ---- Q fragments (B operand of S^T = K Q^T): row qw0 + 16t + r16.
  bf16x8 qf[kRT][4];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const int qpos = qw0 + 16 * t + r16;
    const bool ok = qpos <= qb;
    const uint16_t* src = p.q + (((int64_t)it.b * p.T + (ok ? qpos - P : 0)) * p.hq + qhead) * kD + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ds) : u32x4{0u, 0u, 0u, 0u};
      qf[t][ds] = __builtin_bit_cast(bf16x8, raw);
    }
    if (kFused && p.qpro_on) prologue_frag(qf[t], qpos, g, p.qpro);  // RMSNorm + RoPE of q, once per row
  }

  // ---- key ranges of this work item
  TileRange rg0, rg1;
  int nt0, ntiles;
  {
    KeyRange k0, k1;
    const int nr = prefill_key_ranges(p, it.cls, qa, qb, k0, k1);
    rg0 = TileRange{(int)k0.lo, (int)k0.hi, (int)k0.span, (int)(k0.lo / kPrefillKeys) * kPrefillKeys};
    nt0 = (int)tiles_of(k0);
    ntiles = nt0;
    rg1 = rg0;
    if (nr > 1) {
      rg1 = TileRange{(int)k1.lo, (int)k1.hi, (int)k1.span, (int)(k1.lo / kPrefillKeys) * kPrefillKeys};
      ntiles += (int)tiles_of(k1);
    }
  }
  const TileTest tt0 = tile_test(rg0, qw0, qw1, wave_active);
  const TileTest tt1 = tile_test(rg1, qw0, qw1, wave_active);
  // this workgroup's piece of the unit's tiles (a main unit may be cut into
  // key-range pieces that are merged below; the later pieces of a short unit
  // are empty)
  const PieceRange pr = piece_range(ntiles, it.cls == kMain ? p.n_pieces : 1, it.piece);
  if (pr.t0 >= pr.t1) return;
  const int t_end = pr.t1;
  if (tid == 0) {
    s_fin[0] = it.b;
    s_fin[1] = it.qhead;
    s_fin[2] = qa;
    s_fin[3] = qb;
    s_fin[4] = pr.used;
    s_fin[5] = it.unit;
    s_fin[6] = it.piece;
  }

  KvSrc src;
  src.cstride = (int64_t)p.hkv * kD;
  {
    const int64_t coff = ((int64_t)it.b * p.T * p.hkv + it.kvh) * kD;
    src.ck = p.k + coff;
    src.cv = p.v + coff;
  }
  src.P = P;
  src.cls = it.cls;
  src.ring_cap = p.main_ring ? (int)p.main_cap : 0;
  src.sink = p.sink;
  src.recent = p.recent;
  src.chunk_end = P + p.T;
  if (it.cls == kStream) {
    const int64_t off = ((int64_t)it.b * p.n_stream + it.rank) * (int64_t)(p.sink + p.recent) * kD;
    src.mk = p.k_stream + off;
    src.mv = p.v_stream + off;
  } else {
    const int64_t off = ((int64_t)it.b * p.n_main + it.rank) * p.main_cap * kD;
    src.mk = p.k_main + off;
    src.mv = p.v_main + off;
  }

  // ---- running state (log2 domain: x = s * scale * log2 e)
  const float c = p.scale_log2;
  // thr = m + the rescale threshold and nmu = -m (0 while m is -inf) change
  // only when the maximum moves, so the tile loop reads them ready-made
  float m[kRT], l[kRT], thr[kRT], nmu[kRT];
  f32x4 o[kRT][8];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
    thr[t] = kNegInf;
    nmu[t] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile idx starts at base + 64 idx, with the second range's base moved
  // back by its first tile's index (|values| stay below 2^31)
  const int tb0 = rg0.first, tb1 = rg1.first - kPrefillKeys * nt0;
  auto tile_lo = [&](int idx) { return (idx < nt0 ? tb0 : tb1) + kPrefillKeys * idx; };
  DmaLane dl;
  dl.init(wave, lane);
  auto issue = [&](int idx, uint16_t* dk, uint16_t* dv) {
    const TileRange& r = idx < nt0 ? rg0 : rg1;
    const int lo = tile_lo(idx);
    const TileAddr ta = tile_addr(src, lo);
    dma_tile<false>(dk, src, r, lo, ta, wave, dl);
    dma_tile<true>(dv, src, r, lo, ta, wave, dl);
  };

  // One tile: S^T = K Q^T, then start the next tile's loads into the other
  // buffer, then the softmax and O^T += V^T P^T; wait for this wave's loads
  // and meet at the barrier. Issuing the loads after the QK^T products
  // (rather than first) keeps their LDS writes and scalar address work out
  // of the K-operand reads (2-3% faster on the 4 x 8192 prefill), and the
  // first K fragments are read before the visibility arithmetic so that
  // their LDS latency overlaps it. The other buffer is free from the start
  // of the step: every wave finished reading it before the last barrier.
  auto step = [&](int idx, const uint16_t* cK, const uint16_t* cV, uint16_t* nK, uint16_t* nV) {
    bf16x8 kfirst[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      kfirst[kt] = *reinterpret_cast<const bf16x8*>(&cK[(16 * kt + r16) * kPitch + 8 * (g ^ r16)]);
    const bool first_range = idx < nt0;
    const TileTest tt = first_range ? tt0 : tt1;
    const int lo = tile_lo(idx);
    const bool invisible = lo < tt.vlo || lo > tt.vhi;

    // S^T = K Q^T for 64 keys x 16 kRT rows, and the next tile's load issue,
    // at raised wave priority: the SIMD's other wave is then in its softmax
    // or PV and yields issue slots to these MFMAs (3-4% faster on the
    // 4 x 8192 prefill)
    f32x4 s[kRT][4];
    if (!invisible) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < kRT; ++t)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K fragments one 32-column step ahead of their MFMAs (the fences
      // keep the compiler from regrouping the reads behind full waits)
      bf16x8 kb[2][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) kb[0][kt] = kfirst[kt];
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        if (ds < 3) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            kb[(ds + 1) & 1][kt] =
                *reinterpret_cast<const bf16x8*>(&cK[(16 * kt + r16) * kPitch + 8 * ((4 * (ds + 1) + g) ^ r16)]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int t = 0; t < kRT; ++t) s[t][kt] = mfma_16x16x32(kb[ds & 1][kt], qf[t][ds], s[t][kt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (idx + 1 < t_end) issue(idx + 1, nK, nV);
    __builtin_amdgcn_s_setprio(0);
    if (!invisible) {
      const bool need_mask = lo < tt.mlo || lo > tt.mhi;
      if (need_mask) {
        const TileRange r = first_range ? rg0 : rg1;
        // row q sees keys in [klo, khi]
#pragma unroll
        for (int t = 0; t < kRT; ++t) {
          const int q = qw0 + 16 * t + r16;
          const int klo = max(r.lo, r.span > 0 ? q - r.span + 1 : kNegBig);
          const int khi = min(r.hi, q);
          const int base = lo + 4 * g;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = base + 16 * kt + i;
              if (key < klo || key > khi) s[t][kt][i] = kNegInf;
            }
        }
      }
      // the first V fragments are read before the softmax, whose
      // arithmetic covers their latency; the rest stay 4 steps ahead
      const int s7 = (4 * g + (r16 >> 2)) & 7;  // the V rows' swizzle, the same for every row this lane reads
      const int vrow = (4 * g + (r16 >> 2)) * kVPitch + 4 * (r16 & 3);
      // Each read address is one element offset from the tile array: the
      // compiler tags an LDS access with its array only when the address is
      // a short chain of offsets from it, and an untagged read waits for
      // every load into LDS in flight (the next tile's included).
      i16x4 vr[4][2];
      auto vread = [&](int n, i16x4* d) {
        const int o = vrow + 32 * (n >> 3) * kVPitch + 16 * ((n & 7) ^ s7);
        d[0] = lds_read_tr16(cV + o);
        d[1] = lds_read_tr16(cV + (o + 16 * kVPitch));
      };
#pragma unroll
      for (int n = 0; n < 4; ++n) vread(n, vr[n]);
      __builtin_amdgcn_sched_barrier(0);
      // Online softmax. Each lane holds 16 logits of each of its rows; the
      // 4 lanes of a row share the row maximum. The maximum only moves when
      // some lane's logits exceed it by the rescale threshold, so the
      // cross-lane exchange is skipped on most tiles.
      float lmx[kRT];
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        // chained three-way maxima: 8 instructions for 16 values
        float v = fmaxf(fmaxf(s[t][0][0], s[t][0][1]), s[t][0][2]);
#pragma unroll
        for (int j = 3; j < 15; j += 2)
          v = fmaxf(fmaxf(v, s[t][j >> 2][j & 3]), s[t][(j + 1) >> 2][(j + 1) & 3]);
        v = fmaxf(v, s[t][3][3]);
        lmx[t] = v * c;
      }
      static_assert(kRT == 2, "the rescale test below names both row blocks");
      // one lane mask per row block, or-ed as scalars: a single ballot of the
      // two tests or-ed per lane made the compiler copy the lane mask into a
      // vector register and compare it back (two more vector instructions)
      const uint64_t grow = __builtin_amdgcn_ballot_w64(lmx[0] > thr[0]) | __builtin_amdgcn_ballot_w64(lmx[1] > thr[1]);
      if (grow != 0) {
#pragma unroll
        for (int t = 0; t < kRT; ++t) {
          const float mx = lane4_max(lmx[t]);
          const bool up = mx > m[t] + kRescaleThreshold;
          const float a = up ? fast_exp2(m[t] - mx) : 1.f;
          m[t] = up ? mx : m[t];
          thr[t] = m[t] + kRescaleThreshold;
          nmu[t] = (m[t] == kNegInf) ? 0.f : -m[t];
          l[t] *= a;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[t][dt] *= a;
        }
      }
      bf16x8 pb[kRT][2];
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        float sum;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(__builtin_fmaf(s[t][kt][i], c, nmu[t]));
            s[t][kt][i] = e;
            sum = (kt == 0 && i == 0) ? e : sum + e;
          }
        l[t] += sum;
        pb[t][0] = pack_bf16(s[t][0], s[t][1]);
        pb[t][1] = pack_bf16(s[t][2], s[t][3]);
      }
      // O^T += V^T P^T
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int n = kk * 8 + dt;
          const bf16x8 a = cat_bf16(vr[n & 3][0], vr[n & 3][1]);
          if (n + 4 < 16) vread(n + 4, vr[n & 3]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < kRT; ++t) o[t][dt] = mfma_16x16x32(a, pb[t][kk], o[t][dt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(pr.t0, sK0, sV0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int idx = pr.t0; idx < t_end; idx += 2) {
    step(idx, sK0, sV0, sK1, sV1);
    if (idx + 1 >= t_end) break;
    step(idx + 1, sK1, sV1, sK0, sV0);
  }

  // row sums: the 4 lanes of a row each hold the sum over their own keys
#pragma unroll
  for (int t = 0; t < kRT; ++t) l[t] = lane4_sum(l[t]);

  // The rest reads its parameters afresh from the kernel arguments (at an
  // index the compiler cannot see is 0) and the work item's fields from LDS,
  // where the first thread left them: keeping them in scalar registers across
  // the tile loop spilled scalars there and cost the loop its overlapped LDS
  // reads, and recomputing the work item here cost a chain of dependent
  // scalar steps at every workgroup's end.
  int zero = 0;
  __asm__ volatile("" : "+s"(zero));
  const PrefillParams& pf = (&p)[zero];
  const int fb = __builtin_amdgcn_readfirstlane(s_fin[0]);
  const int fqhead = __builtin_amdgcn_readfirstlane(s_fin[1]);
  const int qaf = __builtin_amdgcn_readfirstlane(s_fin[2]);
  const int qbf = __builtin_amdgcn_readfirstlane(s_fin[3]);
  const int fused = __builtin_amdgcn_readfirstlane(s_fin[4]);
  const int funit = __builtin_amdgcn_readfirstlane(s_fin[5]);
  const int fpiece = __builtin_amdgcn_readfirstlane(s_fin[6]);
  const int qheadf = fqhead + wave / kRowWaves;
  const int Pf = (int)pf.start_pos;
  const int qw0f = qaf + rwave * 16 * kRT;
  const bool wave_activef = qw0f <= qbf;

  // ---- key-range pieces: every piece publishes its partial (running max,
  // sum and unnormalised output, in the accumulator layout) with
  // device-coherent stores, waits for them to complete, and bumps the unit's
  // arrival counter; the last piece to arrive reads all partials back, its
  // own included, and combines them in piece order (max, rescale, add), so
  // the result does not depend on which piece finished last; it finishes the
  // rows below and resets the counter for the next call.
  if (fused > 1) {
    const int gw = pf.group / kHeads;  // workgroups per unit and piece
    const int64_t cslot = (int64_t)funit * gw + (fqhead % pf.group) / kHeads;
    const float* parts = pf.ws_part + cslot * pf.n_pieces * kPartFloats;
    float* mine = pf.ws_part + (cslot * pf.n_pieces + fpiece) * kPartFloats;
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        float* dst = mine + (((wave * kRT + t) * 8 + dt) * 64 + lane) * 4;
        coherent_store2(dst, f32x2{o[t][dt][0], o[t][dt][1]});
        coherent_store2(dst + 2, f32x2{o[t][dt][2], o[t][dt][3]});
      }
      if (g == 0) coherent_store2(mine + kPartOutFloats + ((wave * kRT + t) * 16 + r16) * 2, f32x2{m[t], l[t]});
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int32_t* counter = pf.ws_count + cslot;
    if (tid == 0)
      s_last = (__hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == fused - 1);
    __syncthreads();
    if (!s_last) return;
    for (int q = 0; q < fused; ++q) {
      const float* src = parts + (int64_t)q * kPartFloats;
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        const f32x2 ml = coherent_load2(src + kPartOutFloats + ((wave * kRT + t) * 16 + r16) * 2);
        const float mx = q == 0 ? ml.x : fmaxf(m[t], ml.x);
        const float a = (q == 0 || m[t] == kNegInf) ? 0.f : fast_exp2(m[t] - mx);
        const float b = (ml.x == kNegInf) ? 0.f : (q == 0 ? 1.f : fast_exp2(ml.x - mx));
        m[t] = mx;
        l[t] = (q == 0 ? 0.f : l[t] * a) + ml.y * b;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const float* ps = src + (((wave * kRT + t) * 8 + dt) * 64 + lane) * 4;
          const f32x2 lo = coherent_load2(ps);
          const f32x2 hi = coherent_load2(ps + 2);
          const f32x4 po = f32x4{lo.x, lo.y, hi.x, hi.y};
          o[t][dt] = q == 0 ? po : o[t][dt] * a + po * b;
        }
      }
    }
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!wave_activef) return;
  // ---- epilogue: O = O^T / l (with the attention sink, if any, in l), times
  // the output gate, bf16 round-to-nearest-even; lse = (m + log2 l) ln 2.
  // Each lane holds 4 consecutive columns of a row per 16-column block, so
  // the rows go through LDS (the tile buffers are free after the loop's last
  // barrier; one buffer per wave, 272-byte rows) and leave as whole 256-byte
  // rows, 4 rows per store instruction, instead of 16 scattered 32-byte
  // pieces per instruction.
  constexpr int kOPitch = kD + 8;
  static_assert(kPrefillWaveRows * kOPitch <= kPrefillKeys * kPitch, "staged rows must fit one tile buffer");
  uint16_t* const stage = wave == 0 ? sK0 : (wave == 1 ? sV0 : (wave == 2 ? sK1 : sV1));
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const float lt = l[t];
    const int qpos = qw0f + 16 * t + r16;
    if (qpos > qbf) continue;
    float inv = 1.f / lt;
    const float mu = (m[t] == kNegInf) ? 0.f : m[t];
    float lse = (mu + __log2f(lt)) * kLn2;
    if (kFused && pf.sink_logits != nullptr) {
      const RowNorm rn = row_norm(m[t], lt, pf.sink_logits, qheadf);
      inv = rn.inv;
      lse = rn.lse;
    }
    const int64_t orow = ((int64_t)fb * pf.T + (qpos - Pf)) * pf.hq + qheadf;
    uint16_t* dst = stage + (16 * t + r16) * kOPitch + 4 * g;
    if (!kFused || pf.gate == nullptr) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x4 v = pack_bf16x4(o[t][dt] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    } else if (pf.gate_mode == 2) {
      const float f = inv * gate_factor(bf16_bits_to_f32(pf.gate[orow]));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x4 v = pack_bf16x4(o[t][dt] * f);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    } else {
      const uint16_t* gsrc = pf.gate + orow * kD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint2 gw = *reinterpret_cast<const uint2*>(gsrc + 16 * dt);
        const f32x4 gf = f32x4{gate_factor(bf16_bits_to_f32(gw.x & 0xffffu)), gate_factor(bf16_bits_to_f32(gw.x >> 16)),
                               gate_factor(bf16_bits_to_f32(gw.y & 0xffffu)), gate_factor(bf16_bits_to_f32(gw.y >> 16))};
        const bf16x4 v = pack_bf16x4(o[t][dt] * inv * gf);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    }
    if (pf.lse != nullptr && g == 0) pf.lse[((int64_t)fb * pf.hq + qheadf) * pf.T + (qpos - Pf)] = lse;
  }
  // the wave's own LDS writes are complete before its reads (one wave's LDS
  // operations execute in order)
#pragma unroll
  for (int j = 0; j < kPrefillWaveRows / 4; ++j) {
    const int row = 4 * j + g;
    const int qpos = qw0f + row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * kOPitch + 8 * r16);
    if (qpos <= qbf) {
      const int64_t orow = ((int64_t)fb * pf.T + (qpos - Pf)) * pf.hq + qheadf;
      *reinterpret_cast<u32x4*>(pf.out + orow * kD + 8 * r16) = v;
    }
  }
}

// The plain kernel carries no prologue or epilogue code (1% faster on the
// 4 x 8192 prefill than one kernel that skips it); the fused one is used when
// a call passes a q prologue, sink logits or a gate.
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillParams p) { prefill_body<false, 2>(p); }
__global__ __launch_bounds__(kThreads, 2) void prefill_fused_kernel(PrefillParams p) { prefill_body<true, 2>(p); }
// odd group sizes: 128 rows of one query head per workgroup
__global__ __launch_bounds__(kThreads, 2) void prefill_h1_kernel(PrefillParams p) { prefill_body<false, 1>(p); }
__global__ __launch_bounds__(kThreads, 2) void prefill_h1_fused_kernel(PrefillParams p) { prefill_body<true, 1>(p); }

hipError_t launch_prefill(const PrefillParams& p, int64_t n_blocks, hipStream_t s) {
  const bool fused = p.qpro_on || p.sink_logits != nullptr || p.gate != nullptr;
  auto k = p.hpw == 2 ? (fused ? prefill_fused_kernel : prefill_kernel)
                      : (fused ? prefill_h1_fused_kernel : prefill_h1_kernel);
  hipLaunchKernelGGL(k, dim3((unsigned)n_blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
