// Q/K prologue: RMSNorm of one head's 128 channels, then the rotary position
// embedding (Laguna-XS-2.1 blog post, sliding-window optimisations: q and k
// are RMS-normalised before the rotary embedding; Laguna-M.1-8bit blog post,
// YaRN dynamic RoPE: the rotary parameters of full-attention layers).
//
// Rotation: channel i pairs with channel i + 64 and the pair turns by the
// angle pos * 2 pi * turns[i]: (x_i cos - x_{i+64} sin, x_{i+64} cos + x_i sin),
// both times the attention factor. The per-pair turn rates (YaRN blend
// included) are computed on the host in double precision. On the device the
// angle is reduced in double precision (pos * turns[i] minus its nearest
// integer, so |fraction| <= 1/2 turn at any position below 2^31) and the
// hardware sine/cosine, which take their argument in turns, finish it in
// single precision.
//
// Channel blocks: a lane holds "pair blocks" of 8 channels [8c, 8c + 8) and
// their partners [64 + 8c, 64 + 8c + 8), c in 0..7, so the rotation never
// leaves the lane; the RMS reduction runs over the lanes that share a row.
#pragma once

#include "duo_internal.h"
#include "mfma_common.h"

namespace duo {

__device__ __forceinline__ void unpack8(const bf16x8& v, float (&x)[8]) {
  const u32x4 w = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  return pack_bf16(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]});
}

__device__ __forceinline__ float sumsq8(const float (&x)[8]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = fmaf(x[e], x[e], s);
  return s;
}

// Scale both halves of pair block c by r * w[channel] (RMSNorm once the
// row's mean square is known).
__device__ __forceinline__ void norm_block(float (&lo)[8], float (&hi)[8], int c, float r, const float* w) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    lo[e] *= r * w[8 * c + e];
    hi[e] *= r * w[64 + 8 * c + e];
  }
}

// 1 / sqrt(mean square + eps); an all-zero row with eps = 0 stays zero.
__device__ __forceinline__ float rms_factor(float sumsq, float eps) {
  const float ms = sumsq * (1.f / kD) + eps;
  return ms > 0.f ? __frsqrt_rn(ms) : 0.f;
}

__device__ __forceinline__ void rope_block(float (&lo)[8], float (&hi)[8], int c, int pos, const QkPrologue& pr) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    double t = (double)pos * pr.turns[8 * c + e];
    t -= __builtin_rint(t);
    const float f = (float)t;
    const float sn = __builtin_amdgcn_sinf(f) * pr.attn_factor;
    const float cs = __builtin_amdgcn_cosf(f) * pr.attn_factor;
    const float a = lo[e], b = hi[e];
    lo[e] = a * cs - b * sn;
    hi[e] = b * cs + a * sn;
  }
}

// The prologue on a row held in the MFMA fragment layout of the attention
// kernels: lane (r16, g) holds channels 32 ds + 8 g .. + 7 for ds = 0..3, so
// fragments (0, 2) are pair block g and (1, 3) pair block 4 + g; the four
// lanes g = 0..3 of a row are lanes r16 + 16 g. Every lane of the wave must
// call it (cross-lane reduction).
__device__ __forceinline__ void prologue_frag(bf16x8 (&f)[4], int pos, int g, const QkPrologue& pr) {
  float x[4][8];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) unpack8(f[ds], x[ds]);
  if (pr.norm_w != nullptr) {
    float ss = sumsq8(x[0]) + sumsq8(x[1]) + sumsq8(x[2]) + sumsq8(x[3]);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    const float r = rms_factor(ss, pr.eps);
    norm_block(x[0], x[2], g, r, pr.norm_w);
    norm_block(x[1], x[3], 4 + g, r, pr.norm_w);
  }
  if (pr.rope) {
    rope_block(x[0], x[2], g, pos, pr);
    rope_block(x[1], x[3], 4 + g, pos, pr);
  }
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) f[ds] = pack8(x[ds]);
}

}  // namespace duo
