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
// Workgroup = 4 waves = 128 query rows of one query head; each wave owns 32
// rows as two 16-row MFMA column blocks. Keys come in 64-key tiles over at
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

// LDS row pitches (bf16 elements). K rows are read 16 rows x one 16-byte
// column per instruction (pitch = 4 dwords mod 64 banks keeps them apart);
// V rows are read 4 rows x 32 bytes per 16-lane group by the transpose read
// (pitch = 8 dwords mod 64 keeps those apart).
constexpr int kPitch = kD + 8;    // K: 272 bytes
constexpr int kVPitch = kD + 16;  // V: 288 bytes
constexpr int kNegBig = -0x7fffffff;
// Query rows per wave, in 16-row MFMA column blocks: 32 rows per wave. (64
// rows per wave would halve the LDS operand reads per MFMA, but its
// accumulators and Q fragments do not fit one wave's registers without spills.)
constexpr int kRT = 2;
constexpr int kWaves = kPrefillRows / (16 * kRT);  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
static_assert(kWaves == 4 || kWaves == 8, "4 or 8 waves of 32 rows");

struct TileRange {
  int lo, hi;      // visible key positions of the range (inclusive)
  int span;        // > 0: causal band of this width ending at the query
  int first;       // first tile start (lo rounded down to 64)
};

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

// Addressing of one tile's rows: from one base pointer and a row stride when
// the whole tile lies in the chunk or in a stretch of the cache where
// slot = position, else row by row (positions outside the range clamped onto
// it: their logits are masked, their values are finite data).
struct TileAddr {
  const uint16_t* k;
  const uint16_t* v;
  uint32_t stride_b;  // bytes between consecutive rows (fast form)
  bool general;       // row-by-row form
};

__device__ __forceinline__ TileAddr tile_addr(const KvSrc& s, const TileRange& r, int lo) {
  const int hi = lo + kPrefillKeys - 1;
  const bool inside = lo >= r.lo && hi <= r.hi;
  TileAddr a;
  a.general = false;
  if (inside && lo >= s.P) {
    const int64_t off = (int64_t)(lo - s.P) * s.cstride;
    a.k = s.ck + off;
    a.v = s.cv + off;
    a.stride_b = (uint32_t)s.cstride * 2u;
    return a;
  }
  const bool contiguous_cache = hi < s.P && (s.cls == kStream ? hi < s.sink : s.ring_cap == 0);
  if (inside && contiguous_cache) {
    const int64_t off = (int64_t)lo * kD;
    a.k = s.mk + off;
    a.v = s.mv + off;
    a.stride_b = kD * 2u;
    return a;
  }
  a.k = s.mk;
  a.v = s.mv;
  a.stride_b = 0;
  a.general = true;
  return a;
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS loads of a K (kV = false) or V tile. The padded LDS
// tile is a sequence of 16-byte slots, kSlots per row (16 data columns +
// pad); one load instruction fills 64 consecutive slots, lane l slot 64 j + l,
// and the tile's instructions are dealt round-robin to the waves. A pad
// slot is filled with column 0 of its row (never read). The map holds, for
// each of this wave's instructions, the tile row and the byte offset of the
// column this lane fetches; it is the same for every tile.
template <bool kV>
struct SlotMap {
  static constexpr int kSlots = (kV ? kVPitch : kPitch) / 8;
  static constexpr int kInstr = kPrefillKeys * kSlots / 64;
  static constexpr int kPerWave = (kInstr + kWaves - 1) / kWaves;
  static_assert(kPrefillKeys * kSlots % 64 == 0, "tile must be whole load instructions");
  uint32_t row[kPerWave];
  uint32_t colb[kPerWave];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int jj = 0; jj < kPerWave; ++jj) {
      const int slot = 64 * (wave + kWaves * jj) + lane;
      const int rw = slot / kSlots;
      const int col = slot - rw * kSlots;
      row[jj] = (uint32_t)min(rw, kPrefillKeys - 1);
      colb[jj] = col < 16 ? (uint32_t)col * 16u : 0u;
    }
  }
  __device__ __forceinline__ static bool active(int wave, int jj) {
    return kWaves * (jj + 1) <= kInstr || wave + kWaves * jj < kInstr;
  }
};

template <bool kV>
__device__ __forceinline__ void dma_tile(uint16_t* lds, const KvSrc& s, const TileRange& r, int lo,
                                         const TileAddr& ta, int wave, const SlotMap<kV>& map) {
  uint16_t* dst = lds + wave * 512;
  if (!ta.general) {
    // uniform base + 32-bit lane offset (row < 64, stride < 2^24 bytes)
    const char* base = reinterpret_cast<const char*>(kV ? ta.v : ta.k);
#pragma unroll
    for (int jj = 0; jj < SlotMap<kV>::kPerWave; ++jj) {
      if (SlotMap<kV>::active(wave, jj)) {
        const uint32_t off = __umul24(map.row[jj], ta.stride_b) + map.colb[jj];
        __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void*)(dst + jj * 512 * kWaves), 16, 0, 0);
      }
    }
    return;
  }
#pragma unroll
  for (int jj = 0; jj < SlotMap<kV>::kPerWave; ++jj) {
    if (SlotMap<kV>::active(wave, jj)) {
      int pos = lo + (int)map.row[jj];
      pos = pos < r.lo ? r.lo : (pos > r.hi ? r.hi : pos);
      const Src rs = row_src(s, pos);
      const char* src = reinterpret_cast<const char*>(kV ? rs.v : rs.k) + map.colb[jj];
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + jj * 512 * kWaves), 16, 0, 0);
    }
  }
}

template <bool kFused>
__device__ __forceinline__ void prefill_body(const PrefillParams& p) {
  // Two K/V buffers as separate arrays, so that loads into one are known not
  // to alias reads of the other.
  __shared__ __attribute__((aligned(16))) uint16_t sK0[kPrefillKeys * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[kPrefillKeys * kVPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[kPrefillKeys * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[kPrefillKeys * kVPitch];

  const PrefillItem it = prefill_item(p, blockIdx.x);
  if (!it.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int P = (int)p.start_pos;
  const int last = P + p.T - 1;
  const int qa = P + it.qtile * kPrefillRows;
  const int qb = min(qa + kPrefillRows - 1, last);
  const int qw0 = qa + wave * 16 * kRT;
  const int qw1 = min(qw0 + 16 * kRT - 1, qb);
  const bool wave_active = qw0 <= qb;

  // ---- Q fragments (B operand of S^T = K Q^T): row qw0 + 16t + r16.
  bf16x8 qf[kRT][4];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const int qpos = qw0 + 16 * t + r16;
    const bool ok = qpos <= qb;
    const uint16_t* src = p.q + (((int64_t)it.b * p.T + (ok ? qpos - P : 0)) * p.hq + it.qhead) * kD + 8 * g;
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
  float m[kRT], l[kRT];
  f32x4 o[kRT][8];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto tile_lo = [&](int idx) {
    return idx < nt0 ? rg0.first + kPrefillKeys * idx : rg1.first + kPrefillKeys * (idx - nt0);
  };
  SlotMap<false> kmap;
  SlotMap<true> vmap;
  kmap.init(wave, lane);
  vmap.init(wave, lane);
  auto issue = [&](int idx, uint16_t* dk, uint16_t* dv) {
    const TileRange& r = idx < nt0 ? rg0 : rg1;
    const int lo = tile_lo(idx);
    const TileAddr ta = tile_addr(src, r, lo);
    dma_tile<false>(dk, src, r, lo, ta, wave, kmap);
    dma_tile<true>(dv, src, r, lo, ta, wave, vmap);
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
      kfirst[kt] = *reinterpret_cast<const bf16x8*>(&cK[(16 * kt + r16) * kPitch + 8 * g]);
    const bool first_range = idx < nt0;
    const TileRange r = first_range ? rg0 : rg1;
    const int lo = tile_lo(idx);
    const int hi = lo + kPrefillKeys - 1;
    const bool invisible = !wave_active || lo > qw1 || (r.span > 0 && hi < qw0 - r.span + 1);

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
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 a =
              ds == 0 ? kfirst[kt] : *reinterpret_cast<const bf16x8*>(&cK[(16 * kt + r16) * kPitch + 32 * ds + 8 * g]);
#pragma unroll
          for (int t = 0; t < kRT; ++t) s[t][kt] = mfma_16x16x32(a, qf[t][ds], s[t][kt]);
        }
      }
    }
    if (idx + 1 < ntiles) issue(idx + 1, nK, nV);
    __builtin_amdgcn_s_setprio(0);
    if (!invisible) {
      const bool need_mask = !(lo >= r.lo && hi <= r.hi && hi <= qw0 && (r.span == 0 || lo >= qw1 - r.span + 1));
      if (need_mask) {
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
      // Online softmax. Each lane holds 16 logits of each of its rows; the
      // 4 lanes of a row share the row maximum. The maximum only moves when
      // some lane's logits exceed it by the rescale threshold, so the
      // cross-lane exchange is skipped on most tiles.
      float lmx[kRT];
      bool grow = false;
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        float v = fmaxf(fmaxf(s[t][0][0], s[t][0][1]), fmaxf(s[t][0][2], s[t][0][3]));
#pragma unroll
        for (int kt = 1; kt < 4; ++kt)
          v = fmaxf(fmaxf(v, fmaxf(s[t][kt][0], s[t][kt][1])), fmaxf(s[t][kt][2], s[t][kt][3]));
        lmx[t] = v * c;
        grow = grow || lmx[t] > m[t] + kRescaleThreshold;
      }
      if (__any(grow)) {
#pragma unroll
        for (int t = 0; t < kRT; ++t) {
          float mx = wave_xor_max(lmx[t], 16);
          mx = wave_xor_max(mx, 32);
          const bool up = mx > m[t] + kRescaleThreshold;
          const float a = up ? fast_exp2(m[t] - mx) : 1.f;
          m[t] = up ? mx : m[t];
          l[t] *= a;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) o[t][dt] *= a;
        }
      }
      bf16x8 pb[kRT][2];
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        const float mu = (m[t] == kNegInf) ? 0.f : m[t];
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fast_exp2(__builtin_fmaf(s[t][kt][i], c, -mu));
            s[t][kt][i] = e;
            sum += e;
          }
        l[t] += sum;
        pb[t][0] = pack_bf16(s[t][0], s[t][1]);
        pb[t][1] = pack_bf16(s[t][2], s[t][3]);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* v0 = &cV[(32 * kk + 4 * g + (r16 >> 2)) * kVPitch + 4 * (r16 & 3)];
        const uint16_t* v1 = v0 + 16 * kVPitch;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const bf16x8 a = cat_bf16(lds_read_tr16(v0 + 16 * dt), lds_read_tr16(v1 + 16 * dt));
#pragma unroll
          for (int t = 0; t < kRT; ++t) o[t][dt] = mfma_16x16x32(a, pb[t][kk], o[t][dt]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue(0, sK0, sV0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int idx = 0; idx < ntiles; idx += 2) {
    step(idx, sK0, sV0, sK1, sV1);
    if (idx + 1 >= ntiles) break;
    step(idx + 1, sK1, sV1, sK0, sV0);
  }

  if (!wave_active) return;
  // ---- epilogue: O = O^T / l (with the attention sink, if any, in l), times
  // the output gate, bf16 round-to-nearest-even; lse = (m + log2 l) ln 2
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int qpos = qw0 + 16 * t + r16;
    if (qpos > qb) continue;
    float inv = 1.f / lt;
    const float mu = (m[t] == kNegInf) ? 0.f : m[t];
    float lse = (mu + __log2f(lt)) * kLn2;
    if (kFused && p.sink_logits != nullptr) {
      const RowNorm rn = row_norm(m[t], lt, p.sink_logits, it.qhead);
      inv = rn.inv;
      lse = rn.lse;
    }
    const int64_t orow = ((int64_t)it.b * p.T + (qpos - P)) * p.hq + it.qhead;
    uint16_t* dst = p.out + orow * kD + 4 * g;
    if (!kFused || p.gate == nullptr) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x4 v = pack_bf16x4(o[t][dt] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    } else if (p.gate_mode == 2) {
      const float f = inv * gate_factor(bf16_bits_to_f32(p.gate[orow]));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x4 v = pack_bf16x4(o[t][dt] * f);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    } else {
      const uint16_t* gsrc = p.gate + orow * kD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint2 gw = *reinterpret_cast<const uint2*>(gsrc + 16 * dt);
        const f32x4 gf = f32x4{gate_factor(bf16_bits_to_f32(gw.x & 0xffffu)), gate_factor(bf16_bits_to_f32(gw.x >> 16)),
                               gate_factor(bf16_bits_to_f32(gw.y & 0xffffu)), gate_factor(bf16_bits_to_f32(gw.y >> 16))};
        const bf16x4 v = pack_bf16x4(o[t][dt] * inv * gf);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
      }
    }
    if (p.lse != nullptr && g == 0) p.lse[((int64_t)it.b * p.hq + it.qhead) * p.T + (qpos - P)] = lse;
  }
}

// The plain kernel carries no prologue or epilogue code (1% faster on the
// 4 x 8192 prefill than one kernel that skips it); the fused one is used when
// a call passes a q prologue, sink logits or a gate.
__global__ __launch_bounds__(kThreads, 8 / kWaves) void prefill_kernel(PrefillParams p) { prefill_body<false>(p); }
__global__ __launch_bounds__(kThreads, 8 / kWaves) void prefill_fused_kernel(PrefillParams p) {
  prefill_body<true>(p);
}

hipError_t launch_prefill(const PrefillParams& p, int64_t n_blocks, hipStream_t s) {
  const bool fused = p.qpro_on || p.sink_logits != nullptr || p.gate != nullptr;
  hipLaunchKernelGGL(fused ? prefill_fused_kernel : prefill_kernel, dim3((unsigned)n_blocks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
