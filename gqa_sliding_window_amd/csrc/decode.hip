// Decode attention kernels (gfx950): split-K partials that stream the KV cache
// from HBM, and a merge of the partial softmax states.
//
// One query token per sequence at position L-1 (its K/V already appended).
// Full-context heads read every cached position, streaming heads read their
// sink + recent slots (model card "DuoAttention Laguna Adapter", "Why It
// Works": streaming heads keep only sink tokens plus the most recent tokens),
// a sliding layer reads its window ring (Laguna-M.1-8bit blog post,
// sliding-window section). Every occupied slot of a cache is visible to the
// decode query, so a decode reads slots [0, n) in storage order; softmax does
// not depend on key order.
//
// Partial kernel: one wave per (sequence, KV head, split). The G query heads
// of the KV head are the 16 MFMA columns (G <= 16), so one pass over K/V
// serves the whole group. 32-key tiles are loaded with 16-byte coalesced
// loads, one tile ahead in registers, and go through a wave-private LDS tile
// for the MFMA operand layouts (K row-major, V read transposed).
// Merge kernel: one wave per (sequence, query head) combines the splits with
// the usual max / rescale / sum over partial (m, l, acc).
#include "duo_internal.h"
#include "mfma_common.h"

namespace duo {

constexpr int kDPitch = kD + 8;

// One 32-key tile, global -> registers: rows ld_row + 4 j (clamped to the
// split's last slot), 16-byte chunk ld_chunk; each load instruction of the
// wave covers 4 consecutive 256-byte rows.
__device__ __forceinline__ void load_tile(const uint16_t* kbase, const uint16_t* vbase, int64_t k0,
                                          int64_t k_end, int ld_row, int ld_chunk, u32x4 (&stK)[8],
                                          u32x4 (&stV)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int64_t slot = k0 + ld_row + 4 * j;
    slot = slot < k_end ? slot : k_end - 1;
    stK[j] = *reinterpret_cast<const u32x4*>(kbase + slot * kD + ld_chunk * 8);
    stV[j] = *reinterpret_cast<const u32x4*>(vbase + slot * kD + ld_chunk * 8);
  }
}

__global__ __launch_bounds__(64) void decode_partial_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kDecodeKeys * kDPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kDecodeKeys * kDPitch];

  const DecodeItem it = decode_item(p, blockIdx.x);
  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int g = lane >> 4;

  const int64_t len = p.seq_lens[it.b];
  const int64_t n_valid = decode_valid_slots(p, it.cls, len > 0 ? len : 0);
  const int64_t k_begin = (int64_t)it.split * p.split_keys;
  int64_t k_end = k_begin + p.split_keys;
  if (k_end > n_valid) k_end = n_valid;
  if (k_begin >= k_end) return;  // empty split: the merge does not read it

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

  // Q fragments: column r16 = query head kvh * G + r16 (zero beyond G).
  bf16x8 qf[4];
  {
    const bool ok = r16 < p.group;
    const uint16_t* src = p.q + ((int64_t)it.b * p.hq + it.kvh * p.group + (ok ? r16 : 0)) * kD + 8 * g;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      u32x4 raw = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ds) : u32x4{0u, 0u, 0u, 0u};
      qf[ds] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // staging: rows (lane / 16) + 4 j, chunk lane % 16
  const int ld_row = lane >> 4;
  const int ld_chunk = lane & 15;
  u32x4 stK[8], stV[8];

  const float c = p.scale_log2;
  float m = kNegInf, l = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_tile(kbase, vbase, k_begin, k_end, ld_row, ld_chunk, stK, stV);
  for (int64_t k0 = k_begin; k0 < k_end; k0 += kDecodeKeys) {
    __syncthreads();  // previous tile's LDS reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int off = (ld_row + 4 * j) * kDPitch + ld_chunk * 8;
      *reinterpret_cast<u32x4*>(&sK[off]) = stK[j];
      *reinterpret_cast<u32x4*>(&sV[off]) = stV[j];
    }
    __syncthreads();
    if (k0 + kDecodeKeys < k_end) load_tile(kbase, vbase, k0 + kDecodeKeys, k_end, ld_row, ld_chunk, stK, stV);

    f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sK[(16 * kt + r16) * kDPitch + 32 * ds + 8 * g]);
        s[kt] = mfma_16x16x32(a, qf[ds], s[kt]);
      }
    }
    if (k0 + kDecodeKeys > k_end) {
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
    mx = wave_xor_max(mx, 16);
    mx = wave_xor_max(mx, 32);
    mx *= c;
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
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (r16 >= p.group) return;
  const int h = it.kvh * p.group + r16;
  const int64_t slot = ((int64_t)it.b * p.hq + h) * p.n_split_max + it.split;
  float* acc = p.ws_acc + slot * kD + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(acc + 16 * dt) = o[dt];
  if (g == 0) {
    p.ws_ml[slot * 2 + 0] = m;
    p.ws_ml[slot * 2 + 1] = l;
  }
}

__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= (int64_t)p.batch * p.hq) return;
  const int b = (int)(bh / p.hq);
  const int h = (int)(bh % p.hq);
  const int kvh = h / p.group;
  const int cls = ((p.stream_mask >> kvh) & 1u) ? kStream : kMain;
  const int64_t len = p.seq_lens[b];
  const int64_t n_valid = decode_valid_slots(p, cls, len > 0 ? len : 0);
  int n_used = (int)((n_valid + p.split_keys - 1) / p.split_keys);
  // a length beyond the max_seq_len the grid was planned for is cut to the
  // planned splits (never read past the workspace)
  const int n_planned = (cls == kStream) ? p.n_split_stream : p.n_split_main;
  if (n_used > n_planned) n_used = n_planned;
  uint16_t* dst = p.out + bh * kD + 2 * lane;
  if (n_used == 0) {
    *reinterpret_cast<uint32_t*>(dst) = 0u;
    if (p.lse != nullptr && lane == 0) p.lse[bh] = kNegInf;
    return;
  }
  const float* ml = p.ws_ml + bh * p.n_split_max * 2;
  float M = kNegInf;
  for (int s = 0; s < n_used; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f, a0 = 0.f, a1 = 0.f;
  const float* acc = p.ws_acc + bh * p.n_split_max * kD + 2 * lane;
  for (int s = 0; s < n_used; ++s) {
    const float w = fast_exp2(ml[2 * s] - M);
    L += w * ml[2 * s + 1];
    const float2 v = *reinterpret_cast<const float2*>(acc + (int64_t)s * kD);
    a0 += w * v.x;
    a1 += w * v.y;
  }
  const float inv = 1.f / L;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 r = __builtin_convertvector((f32x2{a0 * inv, a1 * inv}), bf16x2);
  *reinterpret_cast<bf16x2*>(dst) = r;
  if (p.lse != nullptr && lane == 0) p.lse[bh] = (M + __log2f(L)) * kLn2;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.n_items > 0) {
    hipLaunchKernelGGL(decode_partial_kernel, dim3((unsigned)p.n_items), dim3(64), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t waves = (int64_t)p.batch * p.hq;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
