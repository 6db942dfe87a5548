// gfx950 building blocks shared by the attention kernels: bf16 MFMA tiles,
// the LDS transpose read, and bf16 packing.
//
// MFMA layouts used (v_mfma_f32_16x16x32_bf16, wave64; lane l, r = l % 16,
// g = l / 16):
//   A operand (16 x 32):  lane holds A[r][8g .. 8g+7]
//   B operand (32 x 16):  lane holds B[8g .. 8g+7][r]
//   C/D       (16 x 16):  lane holds D[4g .. 4g+3][r]
// Attention is computed transposed, S^T = K Q^T, so that every lane owns one
// query row (column r) and the row's softmax statistics stay in the lane.
// The PV product O^T = V^T P^T takes P^T straight from the S^T registers:
// keys are consumed in the order sigma(8g + j) = 4g + j (j < 4) and
// 16 + 4g + (j - 4) (j >= 4) of each 32-key block, and V^T is read in that
// same order with ds_read_b64_tr_b16, which gives lane i of each 16-lane group
// element i % 4 of the 4-element chunk addressed by lane i / 4 + 4 j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace duo {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 4 x 16 transpose read: lane i of a 16-lane group gets column (i) of the
// 4-row block whose rows the group's lanes address (4 lanes per row, 4
// consecutive bf16 each).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat_bf16(const i16x4& lo, const i16x4& hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& lo, const f32x4& hi) {
  f32x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ bf16x4 pack_bf16x4(const f32x4& v) {
  return __builtin_convertvector(v, bf16x4);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 on the VALU (no LDS
// instruction): each row swap leaves lane l's value and its partner's, in the
// other 16-lane (then 32-lane) half, in the two results.
__device__ __forceinline__ float lane4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over lanes l, l ^ 16, l ^ 32 and l ^ 48, the same way.
__device__ __forceinline__ float lane4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Final normalisation of one output row. M is the row's running maximum in the
// log2 domain (x = scaled logit * log2 e) and L the sum of 2^(x - M) over its
// keys. An attention sink (Laguna-M.1-8bit post, sliding-window optimisations:
// one learnable logit b per query head, natural units) is one more term of the
// softmax denominator whose value row is zero. Returns the factor on the
// unnormalised output and lse = ln(sum e^logit [+ e^b]).
struct RowNorm { float inv, lse; };
__device__ __forceinline__ RowNorm row_norm(float M, float L, const float* sink_logits, int qhead) {
  if (sink_logits == nullptr) return RowNorm{1.f / L, (M + __log2f(L)) * kLn2};
  const float bs = sink_logits[qhead] * kLog2e;
  const float Mn = fmaxf(M, bs);
  const float f = (M == kNegInf) ? 0.f : fast_exp2(M - Mn);
  const float Ln = L * f + fast_exp2(bs - Mn);
  return RowNorm{f / Ln, (Mn + __log2f(Ln)) * kLn2};
}

// Output gate (same post, attention output gating): each output value times
// the logistic function of its gate value.
__device__ __forceinline__ float gate_factor(float g) { return 1.f / (1.f + __expf(-g)); }
// Device-coherent (sc1) stores and loads at agent scope: visible to a
// workgroup on another XCD without writing back or invalidating the L2 caches.
// They carry the split-K partial results between the workgroups of one launch.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats (8-byte aligned) in one device-coherent store / load.
__device__ __forceinline__ void coherent_store2(float* p, f32x2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 coherent_load2(const float* p) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return __builtin_bit_cast(f32x2, v);
}

// Lazy rescaling: the running row maximum is only moved when a new logit
// exceeds it by more than this many powers of two; until then exponentials may
// reach 2^8, far inside fp32 and bf16 range. Output and normaliser share the
// stale maximum, so the result is unchanged.
constexpr float kRescaleThreshold = 8.0f;

}  // namespace duo
