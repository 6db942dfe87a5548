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
// from the k/v inputs.
#include "duo_internal.h"
#include "mfma_common.h"

namespace duo {

constexpr int kPitch = kD + 8;  // LDS row pitch in bf16 elements (272 bytes)

struct RowSrc {
  const uint16_t* k;
  const uint16_t* v;
};

// Address of key position `pos` for (b, kvh): chunk input or cache slot.
__device__ __forceinline__ RowSrc key_row(const PrefillParams& p, const PrefillItem& it,
                                          int64_t pos) {
  RowSrc r;
  if (pos >= p.start_pos) {
    const int64_t off = (((int64_t)it.b * p.T + (pos - p.start_pos)) * p.hkv + it.kvh) * kD;
    r.k = p.k + off;
    r.v = p.v + off;
    return r;
  }
  int64_t off;
  if (it.cls == kStream) {
    const int64_t cap = (int64_t)p.sink + p.recent;
    const int64_t slot = pos < p.sink ? pos : p.sink + (pos - p.sink) % p.recent;
    off = (((int64_t)it.b * p.n_stream + it.rank) * cap + slot) * kD;
    r.k = p.k_stream + off;
    r.v = p.v_stream + off;
  } else {
    const int64_t slot = p.main_ring ? pos % p.main_cap : pos;
    off = (((int64_t)it.b * p.n_main + it.rank) * p.main_cap + slot) * kD;
    r.k = p.k_main + off;
    r.v = p.v_main + off;
  }
  return r;
}

// Tile idx of the (at most two) key ranges: its range and first position.
__device__ __forceinline__ void tile_of(const KeyRange (&rg)[2], int64_t nt0, int64_t idx, KeyRange& r,
                                        int64_t& lo) {
  const bool first = idx < nt0;
  r = first ? rg[0] : rg[1];
  lo = (r.lo / kPrefillKeys + (first ? idx : idx - nt0)) * kPrefillKeys;
}

// Global -> registers: rows ld_row + 16 j of the tile; positions outside the
// range are clamped onto it (their logits are masked, their values finite).
__device__ __forceinline__ void load_tile(const PrefillParams& p, const PrefillItem& it,
                                          const KeyRange (&rg)[2], int64_t nt0, int64_t idx, int ld_row,
                                          int ld_chunk, u32x4 (&stK)[4], u32x4 (&stV)[4]) {
  KeyRange r;
  int64_t lo;
  tile_of(rg, nt0, idx, r, lo);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t pos = lo + ld_row + 16 * j;
    pos = pos < r.lo ? r.lo : (pos > r.hi ? r.hi : pos);
    const RowSrc src = key_row(p, it, pos);
    stK[j] = *reinterpret_cast<const u32x4*>(src.k + ld_chunk * 8);
    stV[j] = *reinterpret_cast<const u32x4*>(src.v + ld_chunk * 8);
  }
}

__device__ __forceinline__ void store_tile(uint16_t* sk, uint16_t* sv, int ld_row, int ld_chunk,
                                           const u32x4 (&stK)[4], const u32x4 (&stV)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int off = (ld_row + 16 * j) * kPitch + ld_chunk * 8;
    *reinterpret_cast<u32x4*>(sk + off) = stK[j];
    *reinterpret_cast<u32x4*>(sv + off) = stV[j];
  }
}

__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kPrefillKeys * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kPrefillKeys * kPitch];

  const PrefillItem it = prefill_item(p, blockIdx.x);
  if (!it.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int64_t P0 = p.start_pos;
  const int64_t qa = P0 + (int64_t)it.qtile * kPrefillRows;
  const int64_t last = P0 + p.T - 1;
  const int64_t qb = (qa + kPrefillRows - 1 < last) ? qa + kPrefillRows - 1 : last;
  const int64_t qw0 = qa + wave * 32;
  const int64_t qw1 = (qw0 + 31 < qb) ? qw0 + 31 : qb;
  const bool wave_active = qw0 <= qb;

  // ---- Q fragments (B operand of S^T = K Q^T): row qw0 + 16t + r16.
  bf16x8 qf[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t qpos = qw0 + 16 * t + r16;
    const bool ok = qpos <= qb;
    const uint16_t* src = p.q + (((int64_t)it.b * p.T + (ok ? qpos - P0 : 0)) * p.hq + it.qhead) * kD + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ds) : u32x4{0u, 0u, 0u, 0u};
      qf[t][ds] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  KeyRange rg[2];
  const int nr = prefill_key_ranges(p, it.cls, qa, qb, rg);
  const int64_t nt0 = tiles_of(rg[0]);
  const int64_t ntiles = nt0 + (nr > 1 ? tiles_of(rg[1]) : 0);

  // ---- per-thread staging of one K/V tile: rows (tid/16) + 16 j, 16-byte chunk tid%16
  const int ld_row = tid >> 4;
  const int ld_chunk = tid & 15;
  u32x4 stK[4], stV[4];

  // ---- running state (log2 domain: x = s * scale * log2 e)
  const float c = p.scale_log2;
  float m[2] = {kNegInf, kNegInf};
  float l[2] = {0.f, 0.f};
  f32x4 o[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(p, it, rg, nt0, 0, ld_row, ld_chunk, stK, stV);
  store_tile(sK[0], sV[0], ld_row, ld_chunk, stK, stV);
  __syncthreads();

  for (int64_t idx = 0; idx < ntiles; ++idx) {
    const int buf = (int)(idx & 1);
    if (idx + 1 < ntiles) load_tile(p, it, rg, nt0, idx + 1, ld_row, ld_chunk, stK, stV);

    KeyRange r;
    int64_t lo;
    tile_of(rg, nt0, idx, r, lo);
    const int64_t hi = lo + kPrefillKeys - 1;
    const bool invisible = !wave_active || lo > qw1 || (r.span > 0 && hi < qw0 - r.span + 1);

    if (!invisible) {
      const bool need_mask = !(lo >= r.lo && hi <= r.hi && hi <= qw0 &&
                               (r.span == 0 || lo >= qw1 - r.span + 1));
      // S^T = K Q^T for 64 keys x 32 rows
      f32x4 s[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) s[t][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[buf][(16 * kt + r16) * kPitch + 32 * ds + 8 * g]);
          s[0][kt] = mfma_16x16x32(a, qf[0][ds], s[0][kt]);
          s[1][kt] = mfma_16x16x32(a, qf[1][ds], s[1][kt]);
        }
      }
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int64_t q = qw0 + 16 * t + r16;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int64_t key = lo + 16 * kt + 4 * g + i;
              const bool vis = key >= r.lo && key <= r.hi && key <= q &&
                               (r.span == 0 || key > q - r.span);
              if (!vis) s[t][kt][i] = kNegInf;
            }
        }
      }
      // online softmax, per row (lane column), stats shared by the 4 lanes of a row
      float mx[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float v = s[t][0][0];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) v = fmaxf(v, s[t][kt][i]);
        v = wave_xor_max(v, 16);
        v = wave_xor_max(v, 32);
        mx[t] = v * c;
      }
      const bool up0 = mx[0] > m[0] + kRescaleThreshold;
      const bool up1 = mx[1] > m[1] + kRescaleThreshold;
      if (__any(up0 || up1)) {
        const float a0 = up0 ? fast_exp2(m[0] - mx[0]) : 1.f;
        const float a1 = up1 ? fast_exp2(m[1] - mx[1]) : 1.f;
        m[0] = up0 ? mx[0] : m[0];
        m[1] = up1 ? mx[1] : m[1];
        l[0] *= a0;
        l[1] *= a1;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          o[0][dt] *= a0;
          o[1][dt] *= a1;
        }
      }
      bf16x8 pb[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
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
        const uint16_t* v0 = &sV[buf][(32 * kk + 4 * g + (r16 >> 2)) * kPitch + 4 * (r16 & 3)];
        const uint16_t* v1 = v0 + 16 * kPitch;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const bf16x8 a = cat_bf16(lds_read_tr16(v0 + 16 * dt), lds_read_tr16(v1 + 16 * dt));
          o[0][dt] = mfma_16x16x32(a, pb[0][kk], o[0][dt]);
          o[1][dt] = mfma_16x16x32(a, pb[1][kk], o[1][dt]);
        }
      }
    }

    if (idx + 1 < ntiles) store_tile(sK[buf ^ 1], sV[buf ^ 1], ld_row, ld_chunk, stK, stV);
    __syncthreads();
  }

  if (!wave_active) return;
  // ---- epilogue: O = O^T / l, bf16 round-to-nearest-even; lse = (m + log2 l) ln 2
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int64_t qpos = qw0 + 16 * t + r16;
    if (qpos > qb) continue;
    const float inv = 1.f / lt;
    const int64_t row = (int64_t)it.b * p.T + (qpos - P0);
    uint16_t* dst = p.out + (row * p.hq + it.qhead) * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const bf16x4 v = pack_bf16x4(o[t][dt] * inv);
      *reinterpret_cast<bf16x4*>(dst + 16 * dt) = v;
    }
    if (p.lse != nullptr && g == 0) {
      const float mu = (m[t] == kNegInf) ? 0.f : m[t];
      p.lse[((int64_t)it.b * p.hq + it.qhead) * p.T + (qpos - P0)] = (mu + __log2f(lt)) * kLn2;
    }
  }
}

hipError_t launch_prefill(const PrefillParams& p, int64_t n_blocks, hipStream_t s) {
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)n_blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
