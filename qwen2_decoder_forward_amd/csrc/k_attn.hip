// Causal grouped-query attention kernels.
//
// Query head h reads KV head h / group (contiguous groups: on the 0.5B shape
// KV head j serves query heads 7j..7j+6, nnterp Qwen2 page, "Grouped-query
// attention"); scores are scaled by head_dim^-0.5; a row at position p sees
// the KV slots 0..p of its own sequence (full causal attention, no window).
// Both kernels load each K/V tile once per KV head and share it across the
// whole query group.
#include "q2_device.h"

namespace q2 {

// ------------------------------------------------------------------ decode
// One block per (split of up to 256 keys, KV head, query row).  A block walks
// its split in 64-key tiles with an online softmax for all `group` query
// heads of the KV head, so each K/V tile is read once per KV head.  With a
// single split the block writes the normalised output itself; otherwise it
// writes (max, exp-sum, un-normalised output) and k_attn_merge combines the
// splits with log-sum-exp rescaling.  No block waits on another.
constexpr int kTile = 64;

struct AttnDecP {
  Dims d;
  int layer;
  KVCache kv;
  const float *q;
  int ldq;
  RowInfo rows;
  AttnPartials part;
  float *o32;
  _Float16 *o16;
  int ldo;
  float scale;
};

template <int HD, bool DIRECT>
__global__ __launch_bounds__(256) void k_attn_decode(AttnDecP p) {
  constexpr int KS = HD + 1;  // padded K row in LDS (conflict-free column walk)
  constexpr int PER = (8 * HD + 255) / 256;
  __shared__ __attribute__((aligned(16))) float sK[kTile * KS];
  __shared__ __attribute__((aligned(16))) float sQ[8 * HD];
  __shared__ float sP[8 * kTile];
  __shared__ float sM[8], sL[8], sA[8];

  const int tid = threadIdx.x;
  const int c = blockIdx.x, g = blockIdx.y, m = blockIdx.z;
  const int G = p.d.group;
  const int pos = p.rows.pos[m];
  const int seq = p.rows.seq[m];
  const int P = pos + 1;
  const int kb = c * kSplitKeys;
  const int ke = min(P, kb + kSplitKeys);
  if (kb >= ke) return;  // uniform across the block

  const float *qrow = p.q + (size_t)m * p.ldq + (size_t)g * G * HD;
  for (int i = tid; i < G * HD; i += 256) sQ[i] = qrow[i] * p.scale;
  if (tid < 8) {
    sM[tid] = kNegInf;
    sL[tid] = 0.f;
  }
  float o[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) o[i] = 0.f;
  const float *kbase = p.kv.k + p.kv.off(p.d, p.layer, seq, g, 0);
  const float *vbase = p.kv.v + p.kv.off(p.d, p.layer, seq, g, 0);
  const int j = tid & 63, wv = tid >> 6;

  for (int k0 = kb; k0 < ke; k0 += kTile) {
    const int nk = min(kTile, ke - k0);
    __syncthreads();
    for (int i = tid * 4; i < nk * HD; i += 1024) {
      const f4 v = *(const f4 *)(kbase + (size_t)k0 * HD + i);
      const int r = i / HD, cc = i - r * HD;
      sK[r * KS + cc + 0] = v.x;
      sK[r * KS + cc + 1] = v.y;
      sK[r * KS + cc + 2] = v.z;
      sK[r * KS + cc + 3] = v.w;
    }
    __syncthreads();
    float s0 = kNegInf, s1 = kNegInf;
    if (j < nk) {
      float a0 = 0.f, a1 = 0.f;
      const bool h1 = wv + 4 < G;
#pragma unroll 8
      for (int dd = 0; dd < HD; ++dd) {
        const float kd = sK[j * KS + dd];
        a0 = fmaf(sQ[wv * HD + dd], kd, a0);
        if (h1) a1 = fmaf(sQ[(wv + 4) * HD + dd], kd, a1);
      }
      s0 = a0;
      s1 = a1;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int h = wv + 4 * i;
      if (h < G) {  // uniform across the wave: wave wv owns heads wv and wv + 4
        const float s = i ? s1 : s0;
        const float m_old = sM[h];
        const float m_new = fmaxf(m_old, wave_max(s));
        const float e = (j < nk) ? __expf(s - m_new) : 0.f;
        const float sum = wave_sum(e);
        sP[h * kTile + j] = e;
        if (j == 0) {
          const float alpha = __expf(m_old - m_new);
          sA[h] = alpha;
          sL[h] = sL[h] * alpha + sum;
          sM[h] = m_new;
        }
      }
    }
    __syncthreads();
    for (int i = tid * 4; i < nk * HD; i += 1024)
      *(f4 *)(sK + i) = *(const f4 *)(vbase + (size_t)k0 * HD + i);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i;
      if (idx < G * HD) {
        const int h = idx / HD, dd = idx - h * HD;
        float acc = o[i] * sA[h];
        for (int jj = 0; jj < nk; ++jj) acc = fmaf(sP[h * kTile + jj], sK[jj * HD + dd], acc);
        o[i] = acc;
      }
    }
  }

  if (DIRECT) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i;
      if (idx < G * HD) {
        const float v = o[i] / sL[idx / HD];
        const size_t oi = (size_t)m * p.ldo + (size_t)g * G * HD + idx;
        if (p.o32) p.o32[oi] = v;
        if (p.o16) p.o16[oi] = (_Float16)v;
      }
    }
  } else {
    const int rec = G * (HD + 2);
    float *part = p.part.buf + (((size_t)m * p.d.nkv + g) * p.part.n_chunks + c) * rec;
    if (tid < G) {
      part[tid] = sM[tid];
      part[G + tid] = sL[tid];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + 256 * i;
      if (idx < G * HD) part[2 * G + idx] = o[i];
    }
  }
}

// Combines the splits of each (row, KV head): O = sum_c e^(m_c - M) o_c /
// sum_c e^(m_c - M) l_c with M the largest split maximum.
template <int HD>
__global__ __launch_bounds__(256) void k_attn_merge(AttnDecP p) {
  const int g = blockIdx.x, m = blockIdx.y;
  const int G = p.d.group;
  const int P = p.rows.pos[m] + 1;
  const int nch = (P + kSplitKeys - 1) / kSplitKeys;
  const int rec = G * (HD + 2);
  const float *base = p.part.buf + ((size_t)m * p.d.nkv + g) * p.part.n_chunks * rec;
  for (int idx = threadIdx.x; idx < G * HD; idx += 256) {
    const int h = idx / HD;
    float mx = kNegInf;
    for (int cc = 0; cc < nch; ++cc) mx = fmaxf(mx, base[(size_t)cc * rec + h]);
    float l = 0.f, acc = 0.f;
    for (int cc = 0; cc < nch; ++cc) {
      const float *r = base + (size_t)cc * rec;
      const float wgt = __expf(r[h] - mx);
      l = fmaf(r[G + h], wgt, l);
      acc = fmaf(r[2 * G + idx], wgt, acc);
    }
    const float v = acc / l;
    const size_t oi = (size_t)m * p.ldo + (size_t)g * G * HD + idx;
    if (p.o32) p.o32[oi] = v;
    if (p.o16) p.o16[oi] = (_Float16)v;
  }
}

template <int HD>
static void attn_decode_hd(const AttnDecP &p, int M, int n_split, hipStream_t st) {
  if (n_split <= 1) {
    hipLaunchKernelGGL((k_attn_decode<HD, true>), dim3(1, p.d.nkv, M), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((k_attn_decode<HD, false>), dim3(n_split, p.d.nkv, M), dim3(256), 0, st, p);
    hipLaunchKernelGGL((k_attn_merge<HD>), dim3(p.d.nkv, M), dim3(256), 0, st, p);
  }
}

void attn_decode(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                 RowInfo rows, int M, int n_split, const AttnPartials &part, float *o32,
                 _Float16 *o16, int ldo, hipStream_t st) {
  AttnDecP p{d, layer, kv, q, ldq, rows, part, o32, o16, ldo, 1.0f / sqrtf((float)d.hd)};
  switch (d.hd) {
    case 16: attn_decode_hd<16>(p, M, n_split, st); break;
    case 64: attn_decode_hd<64>(p, M, n_split, st); break;
    default: attn_decode_hd<128>(p, M, n_split, st); break;
  }
}

// ------------------------------------------------------------------ prefill
// Flash attention on v_mfma_f32_32x32x16_f16, one block per (32-query tile,
// KV head) with one wavefront per query head of the group.  Per 32-key tile:
//   S^T[key, query] = K_tile (A: 32 keys x 16 d) * Q^T (B: 16 d x 32 queries)
// so each lane owns one query column and 16 of the tile's keys (the other 16
// sit in lane ^ 32): the online-softmax max and sum need one cross-lane step,
// and the probabilities are already in the B-operand layout of
//   O^T[d, query] += V^T (A: 32 d x 16 keys) * P^T (B: 16 keys x 32 queries)
// once V^T's key order is matched to the lanes' key order.  K and V are read
// from the f32 cache, rounded to f16 in LDS; accumulation stays in f32.
// MFMA 32x32 operand layout: lane l supplies A[l%32][8*(l/32)..+8] and
// B[8*(l/32)..+8][l%32]; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32], r<16.
struct AttnPreP {
  Dims d;
  int layer;
  KVCache kv;
  const float *q;
  int ldq;
  RowInfo rows;
  int M;
  _Float16 *o16;
  int ldo;
  float qscale;  // head_dim^-0.5 * log2(e): scores in base 2
};

template <int HD>
__global__ __launch_bounds__(512) void k_attn_prefill(AttnPreP p) {
  constexpr int KSTEPS = (HD + 15) / 16;
  constexpr int DT = HD >= 32 ? HD / 32 : 1;  // 32-row d tiles of O^T
  constexpr int DV = DT * 32;
  constexpr int KP = HD + 8;   // padded LDS row of K (halves)
  constexpr int VP = 32 + 8;   // padded LDS row of V^T (halves)
  __shared__ __attribute__((aligned(16))) _Float16 sK[32 * KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[DV * VP];

  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, w = tid >> 6;
  const int G = p.d.group;
  const int tile = gridDim.x - 1 - blockIdx.x;  // longest tiles first
  const int g = blockIdx.y;
  const int h = g * G + w;
  const int r0 = tile * 32;
  const int M = p.M;
  const int last_row = min(r0 + 31, M - 1);
  const int kmax = p.rows.pos[last_row];
  const int seq = p.rows.seq[r0];
  const int qrow = r0 + (lane & 31);
  const bool qvalid = qrow < M;
  const int qpos = qvalid ? p.rows.pos[qrow] : kmax;
  const int hi = lane >> 5;

  if (HD < 32) {
    for (int i = tid; i < DV * VP; i += nthr) sV[i] = (_Float16)0.f;
  }

  h8 qf[KSTEPS];
  {
    const float *qp = p.q + (size_t)(qvalid ? qrow : last_row) * p.ldq + (size_t)h * HD;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qf[s][jj] = (_Float16)(qp[s * 16 + hi * 8 + jj] * p.qscale);
  }

  f16x o[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  const float *kbase = p.kv.k + p.kv.off(p.d, p.layer, seq, g, 0);
  const float *vbase = p.kv.v + p.kv.off(p.d, p.layer, seq, g, 0);
  const int ntiles = kmax / 32 + 1;
  const int n_ctx = p.d.n_ctx;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int key0 = kt * 32;
    __syncthreads();
    for (int i = tid; i < 32 * HD / 4; i += nthr) {
      const int key = (i * 4) / HD, dd = (i * 4) - key * HD;
      f4 kv4 = {0.f, 0.f, 0.f, 0.f}, vv4 = {0.f, 0.f, 0.f, 0.f};
      if (key0 + key < n_ctx) {
        kv4 = *(const f4 *)(kbase + (size_t)(key0 + key) * HD + dd);
        vv4 = *(const f4 *)(vbase + (size_t)(key0 + key) * HD + dd);
      }
      h4 kh = {(_Float16)kv4.x, (_Float16)kv4.y, (_Float16)kv4.z, (_Float16)kv4.w};
      *(h4 *)(sK + key * KP + dd) = kh;
      sV[(dd + 0) * VP + key] = (_Float16)vv4.x;
      sV[(dd + 1) * VP + key] = (_Float16)vv4.y;
      sV[(dd + 2) * VP + key] = (_Float16)vv4.z;
      sV[(dd + 3) * VP + key] = (_Float16)vv4.w;
    }
    __syncthreads();
    if (w >= G) continue;

    f16x s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) {
      h8 a;
      if (HD >= 16) a = *(const h8 *)(sK + (lane & 31) * KP + st * 16 + hi * 8);
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[st], s, 0, 0, 0);
    }
    // causal mask and online softmax (base 2)
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      if (key > qpos) s[r] = kNegInf;
      mt = fmaxf(mt, s[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
    h8 pb0, pb1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = exp2f(s[r] - m_new);
      ls += e;
      if (r < 8) pb0[r] = (_Float16)e;
      else pb1[r - 8] = (_Float16)e;
    }
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
      const _Float16 *vr = sV + (t * 32 + (lane & 31)) * VP;
      h8 a0, a1;
      const h4 x0 = *(const h4 *)(vr + 4 * hi);
      const h4 x1 = *(const h4 *)(vr + 8 + 4 * hi);
      const h4 x2 = *(const h4 *)(vr + 16 + 4 * hi);
      const h4 x3 = *(const h4 *)(vr + 24 + 4 * hi);
      a0 = (h8){x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      a1 = (h8){x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, pb0, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, pb1, o[t], 0, 0, 0);
    }
  }

  if (w >= G || !qvalid) return;
  const float inv_l = 1.0f / l_run;
  _Float16 *orow = p.o16 + (size_t)qrow * p.ldo + (size_t)h * HD;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d0 = t * 32 + 8 * rq + 4 * hi;
      if (d0 < HD) {
        h4 v = {(_Float16)(o[t][4 * rq + 0] * inv_l), (_Float16)(o[t][4 * rq + 1] * inv_l),
                (_Float16)(o[t][4 * rq + 2] * inv_l), (_Float16)(o[t][4 * rq + 3] * inv_l)};
        *(h4 *)(orow + d0) = v;
      }
    }
}

void attn_prefill(const Dims &d, int layer, const KVCache &kv, const float *q, int ldq,
                  RowInfo rows, int M, _Float16 *o16, int ldo, hipStream_t st) {
  AttnPreP p{d, layer, kv, q, ldq, rows, M, o16, ldo,
             (1.0f / sqrtf((float)d.hd)) * 1.4426950408889634f};
  dim3 grid((M + 31) / 32, d.nkv);
  dim3 block(64 * d.group);
  switch (d.hd) {
    case 16: hipLaunchKernelGGL(k_attn_prefill<16>, grid, block, 0, st, p); break;
    case 64: hipLaunchKernelGGL(k_attn_prefill<64>, grid, block, 0, st, p); break;
    default: hipLaunchKernelGGL(k_attn_prefill<128>, grid, block, 0, st, p); break;
  }
}

}  // namespace q2
