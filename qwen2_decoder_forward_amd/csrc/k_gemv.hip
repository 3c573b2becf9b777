// GEMV kernels of the decode path (M <= 8 rows, f32 activations).
//
// Every weight byte is read exactly once per call: a wavefront owns R output
// rows and its 64 lanes stream those rows with 16-byte loads (8 halves per
// lane, 1 KiB per wave instruction), converting binary16 to f32 in registers
// (weights are never expanded in memory).  The activation rows are read
// through the cache by every wave.  Partial sums are reduced across the wave
// with xor shuffles, then the epilogue of the fused op runs on one lane per
// output.  Epilogues:
//   QKV    RMSNorm prologue, bias, RoPE, q write and K/V cache store
//   RESID  h += W x           (WO and down projections)
//   SWIGLU RMSNorm prologue, a = silu(gate) * up on pair-packed rows
//   LMHEAD RMSNorm prologue, logits and greedy argmax (packed 64-bit max)
#include "q2_device.h"

namespace q2 {

enum { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LMHEAD = 3 };

struct GemvP {
  const uint16_t *W;
  int N, K;  // W [N, K], K % 8 == 0
  const float *x;
  int ldx, M;
  const float *norm_w;  // RMSNorm prologue when non-null (width K)
  float eps;
  int n_groups;  // row groups of 4 waves * R rows
  Dims d;
  QkvEpi qkv;
  float *out;
  int ldo;
  ArgmaxEpi am;
  float *normed_out;  // LMHEAD: f32 copy of the normed rows [M, K]
};

template <int MT, int R, int EPI>
__global__ __launch_bounds__(256) void k_gemv(GemvP p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = p.K, M = p.M;

  float inv[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) inv[m] = 1.0f;
  if (EPI != EPI_RESID && p.norm_w) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      if (m < M) {
        float ss = 0.f;
        for (int k = lane * 4; k < K; k += 256) {
          const f4 v = *(const f4 *)(p.x + (size_t)m * p.ldx + k);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
        ss = wave_sum(ss);
        inv[m] = 1.0f / sqrtf(ss / (float)K + p.eps);
      }
    }
  }

  unsigned long long best[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) best[m] = 0ull;

  for (int rg = blockIdx.x; rg < p.n_groups; rg += gridDim.x) {
    const int row0 = (rg * 4 + wave) * R;
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = 0.f;

#pragma unroll 2
    for (int k0 = lane * 8; k0 < K; k0 += 512) {
      h8 wv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int n = row0 + r;
        if (n < p.N)
          wv[r] = __builtin_nontemporal_load((const h8 *)(p.W + (size_t)n * K + k0));
        else
          wv[r] = (h8){0, 0, 0, 0, 0, 0, 0, 0};
      }
      f4 nw0 = {1.f, 1.f, 1.f, 1.f}, nw1 = {1.f, 1.f, 1.f, 1.f};
      if (EPI != EPI_RESID && p.norm_w) {
        nw0 = *(const f4 *)(p.norm_w + k0);
        nw1 = *(const f4 *)(p.norm_w + k0 + 4);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < M) {
          f4 x0 = *(const f4 *)(p.x + (size_t)m * p.ldx + k0);
          f4 x1 = *(const f4 *)(p.x + (size_t)m * p.ldx + k0 + 4);
          if (EPI != EPI_RESID) {
            x0 = x0 * inv[m] * nw0;
            x1 = x1 * inv[m] * nw1;
          }
          const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[r][m] = fmaf((float)wv[r][j], xs[j], acc[r][m]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[r][m] = wave_sum(acc[r][m]);

    if (EPI == EPI_RESID) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < p.N)
            p.out[(size_t)m * p.ldo + row0 + r] += acc[r][m];
    } else if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < p.N)
            p.out[(size_t)m * p.ldo + ((row0 + r) >> 1)] = silu(acc[r][m]) * acc[r + 1][m];
    } else if (EPI == EPI_QKV) {
#pragma unroll
      for (int r = 0; r < R; r += 2)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          if (lane == r * MT + m && m < M && row0 + r < p.N)
            qkv_store_pair(p.d, p.qkv, m, row0 + r, acc[r][m], acc[r + 1][m]);
    } else {  // EPI_LMHEAD
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int n = row0 + r;
          if (m < M && n < p.N) {
            if (p.am.logits && lane == r * MT + m) p.am.logits[(size_t)m * p.N + n] = acc[r][m];
            const unsigned long long key = argmax_key(acc[r][m], n);
            best[m] = key > best[m] ? key : best[m];
          }
        }
    }
  }

  if (EPI == EPI_LMHEAD) {
    __shared__ unsigned long long s_best[4][MT];
    __shared__ int s_last;
    if (lane == 0)
#pragma unroll
      for (int m = 0; m < MT; ++m) s_best[wave][m] = best[m];
    if (blockIdx.x == 0 && wave == 0 && p.normed_out) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M)
          for (int k = lane; k < K; k += 64)
            p.normed_out[(size_t)m * K + k] = p.x[(size_t)m * p.ldx + k] * inv[m] * p.norm_w[k];
    }
    __syncthreads();
    if (threadIdx.x < MT && (int)threadIdx.x < M) {
      const int m = threadIdx.x;
      unsigned long long b = s_best[0][m];
      for (int w = 1; w < 4; ++w) b = s_best[w][m] > b ? s_best[w][m] : b;
      atomicMax(&p.am.best[m], b);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(p.am.counter, 1u) == gridDim.x - 1);
    __syncthreads();
    if (s_last) {
      __threadfence();
      if ((int)threadIdx.x < M) {
        const unsigned long long b = atomicExch(&p.am.best[threadIdx.x], 0ull);
        if (p.am.out) p.am.out[threadIdx.x] = argmax_index(b);
      }
      if (threadIdx.x == 0) atomicExch(p.am.counter, 0u);
    }
  }
}

// ------------------------------------------------------------------ launch
template <int R, int EPI>
static void launch(GemvP &p, int max_grid, hipStream_t st) {
  p.n_groups = (p.N + 4 * R - 1) / (4 * R);
  int grid = p.n_groups < max_grid ? p.n_groups : max_grid;
  if (p.M <= 1)
    hipLaunchKernelGGL((k_gemv<1, R, EPI>), dim3(grid), dim3(256), 0, st, p);
  else if (p.M <= 2)
    hipLaunchKernelGGL((k_gemv<2, R, EPI>), dim3(grid), dim3(256), 0, st, p);
  else if (p.M <= 4)
    hipLaunchKernelGGL((k_gemv<4, R, EPI>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemv<8, R, EPI>), dim3(grid), dim3(256), 0, st, p);
}

static GemvP base(const uint16_t *W, int N, int K, const float *x, int ldx, int M) {
  GemvP p{};
  p.W = W;
  p.N = N;
  p.K = K;
  p.x = x;
  p.ldx = ldx;
  p.M = M;
  return p;
}

void gemv_qkv(const Dims &d, const LayerW &w, const float *h, int M, const QkvEpi &e,
              float eps, hipStream_t st) {
  GemvP p = base(w.wqkv, d.nqkv, d.H, h, d.H, M);
  p.norm_w = w.attn_norm;
  p.eps = eps;
  p.d = d;
  p.qkv = e;
  launch<4, EPI_QKV>(p, 1 << 30, st);
}

void gemv_resid(const uint16_t *W, int N, int K, const float *x, int ldx, int M, float *h,
                int ldh, hipStream_t st) {
  GemvP p = base(W, N, K, x, ldx, M);
  p.out = h;
  p.ldo = ldh;
  if (K >= 2048)
    launch<1, EPI_RESID>(p, 1 << 30, st);
  else
    launch<2, EPI_RESID>(p, 1 << 30, st);
}

void gemv_swiglu(const Dims &d, const LayerW &w, const float *h, int M, float *a, int lda,
                 float eps, hipStream_t st) {
  GemvP p = base(w.wgu, 2 * d.I_pad, d.H, h, d.H, M);
  p.norm_w = w.ffn_norm;
  p.eps = eps;
  p.out = a;
  p.ldo = lda;
  launch<4, EPI_SWIGLU>(p, 1 << 30, st);
}

void gemv_lmhead(const Dims &d, const uint16_t *W, const float *norm_w, const float *h, int M,
                 float *normed_out, const ArgmaxEpi &e, float eps, hipStream_t st) {
  GemvP p = base(W, d.V, d.H, h, d.H, M);
  p.norm_w = norm_w;
  p.eps = eps;
  p.am = e;
  p.normed_out = normed_out;
  launch<4, EPI_LMHEAD>(p, 2048, st);
}

}  // namespace q2
