// Device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q2_kernels.h"

namespace q2 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_huge_valf();

// DPP lane permutations (all rows, all banks): quad_perm [1,0,3,2] and
// [2,3,0,1], row_half_mirror, row_mirror.  They run on the VALU with a few
// cycles of latency, against ~100 for an LDS-routed shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                            0xF, 0xF, true));
}

// Sum over the 64 lanes, result in every lane: four DPP steps combine each
// row of 16 lanes, two shuffles combine the four rows.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
  lo = __shfl_xor(lo, o, 64);
  hi = __shfl_xor(hi, o, 64);
  return ((unsigned long long)hi << 32) | lo;
}

// Greedy readout key: larger logit -> larger key; equal logits -> lower index
// wins; NaN ranks below every number (including -inf) so it never wins; -0
// and +0 compare equal.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  unsigned u = __float_as_uint(v);
  unsigned k;
  if (v != v) k = 0u;
  else if (v == 0.0f) k = 0x80000000u;
  else k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)idx);
}

__device__ __forceinline__ int argmax_index(unsigned long long key) {
  return (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
}

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Fused-QKV epilogue for one packed row pair (n even): adds the bias, rotates
// q and k pairs (NonInterleaved RoPE: packed rows n, n+1 are the natural
// dimensions j and j + hd/2 of one head), then writes q or stores k / v into
// the KV cache slot of row m's sequence at row m's position.
__device__ __forceinline__ void qkv_store_pair(const Dims &d, const QkvEpi &e, int m, int n,
                                               float a, float b) {
  a += e.bias[n];
  b += e.bias[n + 1];
  const int hd = d.hd, half = hd >> 1;
  const int head = n / hd;
  const int j = (n - head * hd) >> 1;
  const int p = e.rows.pos[m];
  if (head < d.nh + d.nkv) {
    const float c = e.rope.cos[(size_t)p * half + j];
    const float s = e.rope.sin[(size_t)p * half + j];
    const float a2 = a * c - b * s;
    const float b2 = b * c + a * s;
    a = a2;
    b = b2;
  }
  float *dst;
  if (head < d.nh) {
    dst = e.q + (size_t)m * e.ldq + (size_t)head * hd;
  } else if (head < d.nh + d.nkv) {
    dst = e.kv.k + e.kv.off(d, e.layer, e.rows.seq[m], head - d.nh, p);
  } else {
    dst = e.kv.v + e.kv.off(d, e.layer, e.rows.seq[m], head - d.nh - d.nkv, p);
  }
  dst[j] = a;
  dst[j + half] = b;
}

}  // namespace q2
