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
// 16-byte loads and stores; the kernel is a pure HBM stream. When a call
// brings more positions than a ring holds, only the newest position of each
// slot is written, so every slot has exactly one writer and the result does
// not depend on scheduling.
#include "duo_internal.h"

namespace duo {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);  // (b, t, kvh)
  const int chunk = threadIdx.x & 15;
  const int64_t rows = (int64_t)p.batch * p.T * p.hkv;
  if (row >= rows) return;
  const int kvh = (int)(row % p.hkv);
  const int64_t bt = row / p.hkv;
  const int t = (int)(bt % p.T);
  const int b = (int)(bt / p.T);
  const int64_t start = p.start_pos[b];
  const int64_t pos = start + t;
  const int64_t end = start + p.T;
  if (pos < 0) return;  // a negative start position writes nothing
  const bool streaming = (p.stream_mask >> kvh) & 1u;
  const int rank = head_rank(p.stream_mask, kvh);

  int64_t slot;
  uint16_t* kdst;
  uint16_t* vdst;
  int64_t head_base;
  if (streaming) {
    if (pos < p.sink) {
      slot = pos;
    } else {
      // newest `recent` non-sink positions of this call only
      const int64_t first = (end - p.recent > p.sink) ? end - p.recent : (int64_t)p.sink;
      if (pos < first) return;
      slot = p.sink + (pos - p.sink) % p.recent;
    }
    head_base = ((int64_t)b * p.n_stream + rank) * (int64_t)(p.sink + p.recent);
    kdst = p.k_stream;
    vdst = p.v_stream;
  } else {
    if (p.main_ring) {
      if (pos < end - p.main_cap) return;  // overwritten later in this call
      slot = pos % p.main_cap;
    } else {
      if (pos >= p.main_cap) return;       // outside the caller's buffer
      slot = pos;
    }
    head_base = ((int64_t)b * p.n_main + rank) * p.main_cap;
    kdst = p.k_main;
    vdst = p.v_main;
  }
  const int64_t src = row * kD + chunk * 8;
  const int64_t dst = (head_base + slot) * kD + chunk * 8;
  const uint4 kv = *reinterpret_cast<const uint4*>(p.k_new + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(p.v_new + src);
  *reinterpret_cast<uint4*>(kdst + dst) = kv;
  *reinterpret_cast<uint4*>(vdst + dst) = vv;
}

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.batch * p.T * p.hkv;
  const int64_t blocks = (rows + 15) / 16;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace duo
