// Device-side helpers shared by the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q2_kernels.h"

namespace q2 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
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

// The two values a lane pair (l, l ^ 16) or (l, l ^ 32) holds, in both lanes
// of the pair: v_permlane16_swap / v_permlane32_swap with the same register
// as both operands return the even and the odd row (half) of the pair.
// They run on the VALU, against an LDS round trip for a shuffle.
__device__ __forceinline__ void pair16(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), true, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), true, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum32(float v) {  // v[l] + v[l ^ 32]
  float a, b;
  pair32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float max32(float v) {  // max(v[l], v[l ^ 32])
  float a, b;
  pair32(v, a, b);
  return fmaxf(a, b);
}

// Sum over the 64 lanes, result in every lane: four DPP steps combine each
// row of 16 lanes, two lane-pair swaps combine the four rows.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  float a, b;
  pair16(v, a, b);
  return sum32(a + b);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  v = fmaxf(v, dpp<0x140>(v));
  float a, b;
  pair16(v, a, b);
  return max32(fmaxf(a, b));
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
// the KV cache slot of row m's sequence at row m's position.  Split in two so
// a kernel can issue the loads the epilogue needs (position, sequence slot,
// bias, then cos/sin of the position) long before its sums are ready.
struct QkvPair {
  float *dst;      // element j of the q row or KV cache slot (j + hd/2 is the partner)
  _Float16 *d16;   // the same element in the binary16 mirror (k, v only)
  int stride16;    // mirror distance from element j to j + hd/2
  float ba, bb;    // bias of the two rows
  float c, s;      // rotation (1, 0 for v)
  int half;
};

// Vector-memory load of a value that would otherwise become a scalar load:
// vector loads complete in issue order, so one issued before a kernel's
// weight stream can be waited for without waiting for the stream, while a
// scalar load's result would be waited for before the stream is issued.
// Loaded as unsigned: widening it to 64 bits (done next to the load by the
// compiler) is then a zero-extension that does not wait for the value.
// The index is passed through an empty asm in a vector register, so the
// value counts as per-lane and is not moved to a scalar register (which
// would also wait for it right away); the base keeps its global address
// space, so the load stays a global (not flat) load.
__device__ __forceinline__ unsigned vload(const int *base, int i) {
  asm volatile("" : "+v"(i));
  return __hip_atomic_load((const unsigned *)base + i, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
}

// First half: the position / sequence loads (no dependent loads yet).
__device__ __forceinline__ void qkv_pair_begin(const QkvEpi &e, int m, int n, unsigned &pos,
                                               unsigned &seq, float &ba, float &bb) {
  pos = vload(e.rows.pos, m);
  seq = vload(e.rows.seq, m);
  ba = e.bias[n];
  bb = e.bias[n + 1];
}

// Second half: destination address and the cos/sin loads, given the position.
__device__ __forceinline__ QkvPair qkv_pair_end(const Dims &d, const QkvEpi &e, int m, int n,
                                                unsigned pos, unsigned seq, float ba, float bb) {
  const int hd = d.hd, half = hd >> 1;
  const int head = n / hd;
  const int j = (n - head * hd) >> 1;
  QkvPair q;
  q.ba = ba;
  q.bb = bb;
  q.half = half;
  q.c = 1.0f;
  q.s = 0.0f;
  if (head < d.nh + d.nkv) {
    q.c = e.rope.cos[(size_t)pos * half + j];
    q.s = e.rope.sin[(size_t)pos * half + j];
  }
  // KV slot offset as in KVCache::off, with the (non-negative) sequence and
  // position widened as unsigned values
  const bool is_k = head < d.nh + d.nkv;
  const size_t g = (size_t)(is_k ? head - d.nh : head - d.nh - d.nkv);
  const size_t blk = ((size_t)e.layer * d.n_seq + (size_t)seq) * d.nkv + g;
  const size_t slot = (blk * d.n_ctx + (size_t)pos) * (size_t)hd + (size_t)j;
  const size_t b16 = blk * (size_t)e.kv.ldp * hd;
  q.d16 = nullptr;
  q.stride16 = 0;
  if (head < d.nh) {
    q.dst = e.q + (size_t)m * e.ldq + (size_t)head * hd + j;
  } else if (is_k) {
    q.dst = e.kv.k + slot;
    q.d16 = e.kv.k16 + b16 + (size_t)pos * hd + j;
    q.stride16 = half;
  } else {
    q.dst = e.kv.v + slot;
    q.d16 = e.kv.v16t + b16 + (size_t)j * e.kv.ldp + pos;
    q.stride16 = half * e.kv.ldp;
  }
  return q;
}

__device__ __forceinline__ void qkv_pair_store(const QkvPair &q, float a, float b) {
  a += q.ba;
  b += q.bb;
  const float x = a * q.c - b * q.s, y = b * q.c + a * q.s;
  q.dst[0] = x;
  q.dst[q.half] = y;
  if (q.d16) {
    q.d16[0] = (_Float16)x;
    q.d16[q.stride16] = (_Float16)y;
  }
}

__device__ __forceinline__ void qkv_store_pair(const Dims &d, const QkvEpi &e, int m, int n,
                                               float a, float b) {
  unsigned pos, seq;
  float ba, bb;
  qkv_pair_begin(e, m, n, pos, seq, ba, bb);
  qkv_pair_store(qkv_pair_end(d, e, m, n, pos, seq, ba, bb), a, b);
}

// Marks loaded values as used here, so the compiler cannot sink their loads
// into the (predicated) blocks that consume them: loads sunk between stores
// are each waited for, together with every store before them.
template <typename T, int N>
__device__ __forceinline__ void pin_regs(T (&a)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(a[i]));
}

// The same epilogue for NE rows m[] (valid row indices) of one packed column
// pair (n even, n + 1 < nqkv).  Every load of the NE rows (position and
// sequence slot, then cos / sin at those positions) is issued before any
// store, so the loads cost two memory round trips in all.  The stores go
// out in groups of GS rows whose values and addresses are all computed
// first: a register written after a store that reads it makes the compiler
// wait for that store to complete (s_waitcnt vmcnt), so this bounds those
// waits to one per group.  Rows with ok[] false store nothing.
template <int NE, int GS = 4>
__device__ __forceinline__ void qkv_store_rows(const Dims &d, const QkvEpi &e, const int (&m)[NE],
                                               int n, const float (&a)[NE], const float (&b)[NE],
                                               const bool (&ok)[NE]) {
  static_assert(NE % GS == 0, "groups of GS rows");
  unsigned pos[NE], seq[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    pos[k] = (unsigned)e.rows.pos[m[k]];
    seq[k] = (unsigned)e.rows.seq[m[k]];
  }
  float bias[2] = {e.bias[n], e.bias[n + 1]};
  const int hd = d.hd, half = hd >> 1;
  const int head = n / hd;
  const int j = (n - head * hd) >> 1;
  const bool rot = head < d.nh + d.nkv;
  float cs[NE], sn[NE];
#pragma unroll
  for (int k = 0; k < NE; ++k) {
    const float c = e.rope.cos[(size_t)pos[k] * half + j];
    const float s = e.rope.sin[(size_t)pos[k] * half + j];
    cs[k] = rot ? c : 1.0f;
    sn[k] = rot ? s : 0.0f;
  }
  pin_regs(seq);
  pin_regs(cs);
  pin_regs(sn);
  pin_regs(bias);
  const bool is_q = head < d.nh, is_k = !is_q && rot;
  const size_t g = (size_t)(is_k ? head - d.nh : head - d.nh - d.nkv);
  const size_t s16 = is_k ? (size_t)half : (size_t)half * e.kv.ldp;  // mirror partner distance
#pragma unroll
  for (int k0 = 0; k0 < NE; k0 += GS) {
    float xs[GS], ys[GS];
    float *p0[GS], *p1[GS];
    _Float16 *q0[GS], *q1[GS];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int k = k0 + u;
      const float x0 = a[k] + bias[0], y0 = b[k] + bias[1];
      xs[u] = x0 * cs[k] - y0 * sn[k];
      ys[u] = y0 * cs[k] + x0 * sn[k];
      const size_t blk = ((size_t)e.layer * d.n_seq + (size_t)seq[k]) * d.nkv + g;
      const size_t slot = (blk * d.n_ctx + (size_t)pos[k]) * (size_t)hd + (size_t)j;
      const size_t b16 = blk * (size_t)e.kv.ldp * hd;
      float *dst = is_q ? e.q + (size_t)m[k] * e.ldq + (size_t)head * hd + j
                        : (is_k ? e.kv.k : e.kv.v) + slot;
      _Float16 *d16 = is_k ? e.kv.k16 + b16 + (size_t)pos[k] * hd + j
                           : e.kv.v16t + b16 + (size_t)j * e.kv.ldp + pos[k];
      p0[u] = dst;
      p1[u] = dst + half;
      q0[u] = d16;
      q1[u] = d16 + s16;
    }
    pin_regs(xs);
    pin_regs(ys);
    pin_regs(p0);
    pin_regs(p1);
    pin_regs(q0);
    pin_regs(q1);
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      if (!ok[k0 + u]) continue;
      *p0[u] = xs[u];
      *p1[u] = ys[u];
      if (!is_q) {
        *q0[u] = (_Float16)xs[u];
        *q1[u] = (_Float16)ys[u];
      }
    }
  }
}


// A producer block of an L2Warm (linear block id bid) reads its share of the
// groups the later launch reads on this XCD: the XCD's groups g = x + 8 t
// are split into contiguous runs of t over the XCD's producers, and the
// run is read flat, 256 threads x 16 bytes a step, every step issued before
// any is waited for (steps past the run are skipped, block-uniformly; a
// thread's part of the last step that falls past the run or the matrix
// reloads the matrix's first 16 bytes).  The loaded words feed an empty asm
// only.
template <int NL>  // at most NL steps per producer (the host plans for that)
__device__ __forceinline__ void l2_warm(const L2Warm &f, int bid) {
  const int x = bid & 7;
  const int first = f.p0 + ((x - f.p0) & 7);  // this XCD's first producer
  const int n_x = (f.p0 + f.n_prod - first + 7) >> 3;
  const int j = (bid - first) >> 3;
  const int T = (f.n_groups - x + 7) >> 3;  // groups the later launch reads on this XCD
  const int t1 = (int)((long long)(j + 1) * T / n_x);
  int t = (int)((long long)j * T / n_x), e = threadIdx.x;
  const int steps = ((t1 - t) * f.group_u4 + 255) >> 8;  // (block-uniform)
  uint4 v[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    v[i] = (uint4){0u, 0u, 0u, 0u};
    if (i < steps) {
      long long a = (long long)(x + 8 * t) * f.group_u4 + e;
      if (t >= t1 || a >= f.total_u4) a = 0;
      v[i] = f.base[a];
      e += 256;
      if (e >= f.group_u4) {  // (group_u4 >= 256: at most one group per step)
        e -= f.group_u4;
        ++t;
      }
    }
  }
  unsigned acc = 0;
#pragma unroll
  for (int i = 0; i < NL; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  asm volatile("" ::"v"(acc));
}

}  // namespace q2
