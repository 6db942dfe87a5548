// KV append: copy new K/V rows into the layer's static cache.
//
// Cache placement (the pages never describe slots; this is the library's
// contract, stated in duo_attn.h): full-context heads of a full layer keep
// every position (slot = position), a sliding layer keeps a ring of W slots,
// streaming heads keep the sink positions and a ring of `recent` slots
// (model card "DuoAttention Laguna Adapter", "Summary" and "Why It Works":
// streaming heads hold the first positions of the sequence and a window of
// the newest ones).
//
// One 256-byte row (one token of one KV head) is copied by 16 lanes with
// 16-byte loads and stores; the kernel is a pure HBM stream. With a k
// prologue (RMSNorm + rotary embedding, see qk_prologue.h) K is transformed
// on its way into the cache; V is always a bit copy. When a call
// brings more positions than a ring holds, only the newest position of each
// slot is written, so every slot has exactly one writer and the result does
// not depend on scheduling.
#include "duo_internal.h"
#include "qk_prologue.h"

namespace duo {

// Destination of row (b, t, kvh): the cache row offset (elements) and the
// K/V caches it lies in; false when this call does not write the row.
struct AppendDst {
  uint16_t* k;
  uint16_t* v;
  int64_t off;
  int pos;
};

// Positions dropped for lying past a contiguous main cache (duo_device_errors),
// one word per device.
__device__ unsigned int g_append_errors;

// `lead`: the one lane of the row that records a dropped position.
__device__ __forceinline__ bool append_dst(const AppendParams& p, int64_t row, bool lead, AppendDst& d) {
  const int kvh = (int)(row % p.hkv);
  const int64_t bt = row / p.hkv;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  const int64_t start = p.start_pos[b];
  const int64_t pos = start + t;
  const int64_t end = start + p.T;
  if (pos < 0) return false;  // a negative start position writes nothing
  const bool streaming = (p.stream_mask >> kvh) & 1u;
  const int rank = head_rank(p.stream_mask, kvh);

  int64_t slot, head_base;
  if (streaming) {
    if (pos < p.sink) {
      slot = pos;
    } else {
      // newest `recent` non-sink positions of this call only
      const int64_t first = (end - p.recent > p.sink) ? end - p.recent : (int64_t)p.sink;
      if (pos < first) return false;
      slot = p.sink + (pos - p.sink) % p.recent;
    }
    head_base = ((int64_t)b * p.n_stream + rank) * (int64_t)(p.sink + p.recent);
    d.k = p.k_stream;
    d.v = p.v_stream;
  } else {
    if (p.main_ring) {
      if (pos < end - p.main_cap) return false;  // overwritten later in this call
      slot = pos % p.main_cap;
    } else {
      if (pos >= p.main_cap) {                   // outside the caller's buffer
        if (lead) atomicOr(&g_append_errors, kDevAppendPastCapacity);
        return false;
      }
      slot = pos;
    }
    head_base = ((int64_t)b * p.n_main + rank) * p.main_cap;
    d.k = p.k_main;
    d.v = p.v_main;
  }
  d.off = (head_base + slot) * kD;
  d.pos = (int)pos;
  return true;
}

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, kvh)
  const int chunk = threadIdx.x & 15;
  if (row >= (int64_t)p.batch * p.T * p.hkv) return;
  AppendDst d;
  if (!append_dst(p, row, chunk == 0, d)) return;
  const int64_t src = row * kD + chunk * 8;
  const uint4 kv = *reinterpret_cast<const uint4*>(p.k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(p.v_new + src);
  *reinterpret_cast<uint4*>(d.k + d.off + chunk * 8) = kv;
  *reinterpret_cast<uint4*>(d.v + d.off + chunk * 8) = vv;
}

// With the k prologue: 8 lanes per row, lane c holding pair block c
// (channels [8c, 8c + 8) and [64 + 8c, 64 + 8c + 8)), so the rotation stays
// in the lane and the RMS sum is a reduction over the row's 8 lanes. The 8
// lanes of a row take the same branch, so a skipped row never feeds the
// reduction of a written one.
__global__ __launch_bounds__(256) void kv_append_pro_kernel(AppendParams p) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  if (row >= (int64_t)p.batch * p.T * p.hkv) return;
  AppendDst d;
  if (!append_dst(p, row, c == 0, d)) return;
  const int64_t src = row * kD + 8 * c;
  float lo[8], hi[8];
  unpack8(*reinterpret_cast<const bf16x8*>(p.k_new + src), lo);
  unpack8(*reinterpret_cast<const bf16x8*>(p.k_new + src + 64), hi);
  const uint4 v0 = *reinterpret_cast<const uint4*>(p.v_new + src);
  const uint4 v1 = *reinterpret_cast<const uint4*>(p.v_new + src + 64);
  if (p.kpro.norm_w != nullptr) {
    float ss = sumsq8(lo) + sumsq8(hi);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    norm_block(lo, hi, c, rms_factor(ss, p.kpro.eps), p.kpro.norm_w);
  }
  if (p.kpro.rope) rope_block(lo, hi, c, d.pos, p.kpro);
  *reinterpret_cast<bf16x8*>(d.k + d.off + 8 * c) = pack8(lo);
  *reinterpret_cast<bf16x8*>(d.k + d.off + 64 + 8 * c) = pack8(hi);
  *reinterpret_cast<uint4*>(d.v + d.off + 8 * c) = v0;
  *reinterpret_cast<uint4*>(d.v + d.off + 64 + 8 * c) = v1;
}

// Standalone prologue, y = prologue(x) row by row (x == y allowed): row
// (b, t, h) of [B, T, H, 128] at position start_pos[b] + t. Same lane layout
// as kv_append_pro_kernel.
__global__ __launch_bounds__(256) void qk_prologue_kernel(PrologueParams p) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int c = threadIdx.x & 7;
  if (row >= (int64_t)p.batch * p.T * p.heads) return;
  const int64_t bt = row / p.heads;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  const int pos = p.start_pos[b] + t;
  const int64_t src = row * kD + 8 * c;
  float lo[8], hi[8];
  unpack8(*reinterpret_cast<const bf16x8*>(p.x + src), lo);
  unpack8(*reinterpret_cast<const bf16x8*>(p.x + src + 64), hi);
  if (p.pr.norm_w != nullptr) {
    float ss = sumsq8(lo) + sumsq8(hi);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    ss += __shfl_xor(ss, 4);
    norm_block(lo, hi, c, rms_factor(ss, p.pr.eps), p.pr.norm_w);
  }
  if (p.pr.rope) rope_block(lo, hi, c, pos, p.pr);
  *reinterpret_cast<bf16x8*>(p.y + src) = pack8(lo);
  *reinterpret_cast<bf16x8*>(p.y + src + 64) = pack8(hi);
}

hipError_t append_device_errors(uint32_t* bits, bool clear) {
  unsigned v = 0u;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_append_errors), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear && v != 0u) {
    const unsigned z = 0u;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_append_errors), &z, sizeof z, 0, hipMemcpyHostToDevice);
  }
  *bits |= v;
  return e;
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.T * p.hkv;
  if (prologue_active(p.kpro)) {
    hipLaunchKernelGGL(kv_append_pro_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_qk_prologue(const PrologueParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.T * p.heads;
  if (rows > 0) hipLaunchKernelGGL(qk_prologue_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
