// MFMA GEMM of the prefill and batched-decode projections:
//   C[M, N] = A[M, K] * W[N, K]^T,  A and W binary16, f32 accumulation,
// on v_mfma_f32_32x32x16_f16.  Block tile 128 x 128 x 32, four wavefronts in
// a 2 x 2 arrangement, each owning 64 x 64 (2 x 2 MFMA tiles).  The next K
// slice is fetched into registers while the current one is multiplied out of
// LDS.  Epilogues are fused:
//   QKV    bias + RoPE + q write / K,V cache store (pair partner via lane^1)
//   RESID  h += C                (WO, down)
//   SWIGLU a = silu(gate) * up   (pair-packed gate/up rows, f16 out)
//   LMHEAD logits + per-row greedy argmax
// MFMA 32x32 layout: lane l supplies A[l%32][8*(l/32)..+8] and
// B[8*(l/32)..+8][l%32]; it receives D[8*(r/4) + 4*(l/32) + r%4][l%32].
#include "q2_device.h"

namespace q2 {

enum { G_QKV = 0, G_RESID = 1, G_SWIGLU = 2, G_LMHEAD = 3 };

constexpr int BM = 128, BN = 128, BK = 32, LDT = BK + 8;
constexpr int kStages = 4;  // K slices in flight per block

struct GemmP {
  const _Float16 *A;
  int lda, M;
  const _Float16 *W;
  int N, K;
  Dims d;
  QkvEpi qkv;
  float *h;
  int ldh;
  _Float16 *a16;
  int ld_a;
  ArgmaxEpi am;
  float *ws;      // split-K: raw partial sums [splits][M][N] (epilogue runs later)
  int k_steps;    // K slices of BK per split
};

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmP p) {
  __shared__ __attribute__((aligned(16))) _Float16 sA[BM * LDT];
  __shared__ __attribute__((aligned(16))) _Float16 sW[BN * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int hi = lane >> 5, l32 = lane & 31;

  // each thread moves two 16-byte chunks of A and two of W per K slice
  const int cr0 = tid >> 2, cr1 = (tid + 256) >> 2, ck = (tid & 3) * 8;
  const bool a0ok = m0 + cr0 < M, a1ok = m0 + cr1 < M;
  const bool w0ok = n0 + cr0 < N, w1ok = n0 + cr1 < N;
  const _Float16 *Ap0 = p.A + (size_t)(a0ok ? m0 + cr0 : 0) * p.lda + ck;
  const _Float16 *Ap1 = p.A + (size_t)(a1ok ? m0 + cr1 : 0) * p.lda + ck;
  const _Float16 *Wp0 = p.W + (size_t)(w0ok ? n0 + cr0 : 0) * K + ck;
  const _Float16 *Wp1 = p.W + (size_t)(w1ok ? n0 + cr1 : 0) * K + ck;
  const h8 zero = {0, 0, 0, 0, 0, 0, 0, 0};

  f16x acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // K slices kt0 .. kt0 + nk - 1; a ring of kStages register sets keeps the
  // global loads of the next kStages - 1 slices in flight while one slice is
  // multiplied out of LDS.
  const int kt0 = blockIdx.z * p.k_steps;
  const int nk = min(K / BK - kt0, p.k_steps);
  h8 ra[kStages][2], rw[kStages][2];
#pragma unroll
  for (int st = 0; st < kStages; ++st) {
    const int ko = (kt0 + st) * BK;
    const bool ok = st < nk;
    ra[st][0] = ok && a0ok ? *(const h8 *)(Ap0 + ko) : zero;
    ra[st][1] = ok && a1ok ? *(const h8 *)(Ap1 + ko) : zero;
    rw[st][0] = ok && w0ok ? *(const h8 *)(Wp0 + ko) : zero;
    rw[st][1] = ok && w1ok ? *(const h8 *)(Wp1 + ko) : zero;
  }
  for (int kb = 0; kb < nk; kb += kStages) {
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      const int kt = kb + st;
      if (kt < nk) {  // uniform across the block
        *(h8 *)(sA + cr0 * LDT + ck) = ra[st][0];
        *(h8 *)(sA + cr1 * LDT + ck) = ra[st][1];
        *(h8 *)(sW + cr0 * LDT + ck) = rw[st][0];
        *(h8 *)(sW + cr1 * LDT + ck) = rw[st][1];
        __syncthreads();
        const int kn = kt + kStages;
        if (kn < nk) {
          const int ko = (kt0 + kn) * BK;
          ra[st][0] = a0ok ? *(const h8 *)(Ap0 + ko) : zero;
          ra[st][1] = a1ok ? *(const h8 *)(Ap1 + ko) : zero;
          rw[st][0] = w0ok ? *(const h8 *)(Wp0 + ko) : zero;
          rw[st][1] = w1ok ? *(const h8 *)(Wp1 + ko) : zero;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          h8 af[2], bf[2];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            af[i] = *(const h8 *)(sA + (wm * 64 + i * 32 + l32) * LDT + s * 16 + hi * 8);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            bf[j] = *(const h8 *)(sW + (wn * 64 + j * 32 + l32) * LDT + s * 16 + hi * 8);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
      }
    }
  }

  // ---------------------------------------------------------------- epilogue
  if (p.ws) {  // split-K: store the raw partial sums
    float *ws = p.ws + (size_t)blockIdx.z * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (m < M && n < N) ws[(size_t)m * N + n] = acc[i][j][r];
        }
      }
    return;
  }
  if (EPI == G_LMHEAD) {
    __shared__ unsigned long long sBest[2][BM];
    float *logits = *p.am.logits;
    unsigned long long kb[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        unsigned long long b = 0ull;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + wn * 64 + j * 32 + l32;
          if (m < M && n < N) {
            const float v = acc[i][j][r];
            if (logits) logits[(size_t)m * N + n] = v;
            const unsigned long long key = argmax_key(v, n);
            b = key > b ? key : b;
          }
        }
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
          const unsigned long long x = shfl_xor_u64(b, o);
          b = x > b ? x : b;
        }
        kb[i][r] = b;
      }
    if (l32 == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) sBest[wn][wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)] = kb[i][r];
    }
    __syncthreads();
    if (tid < BM && m0 + tid < M) {
      const unsigned long long b = sBest[0][tid] > sBest[1][tid] ? sBest[0][tid] : sBest[1][tid];
      atomicMax(&p.am.best[m0 + tid], b);
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const float v = acc[i][j][r];
        if (EPI == G_RESID) {
          if (m < M && n < N) p.h[(size_t)m * p.ldh + n] += v;
        } else {
          const float partner = __shfl_xor(v, 1, 64);
          if ((n & 1) == 0 && m < M && n < N) {
            if (EPI == G_QKV)
              qkv_store_pair(p.d, p.qkv, m, n, v, partner);
            else
              p.a16[(size_t)m * p.ld_a + (n >> 1)] = (_Float16)(silu(v) * partner);
          }
        }
      }
    }
}

// Split-K epilogue: sums the partials of a column pair and applies the op.
template <int EPI>
__global__ __launch_bounds__(256) void k_splitk_epi(GemmP p, int splits) {
  const int M = p.M, N = p.N;
  const int half = N >> 1;
  for (int t = blockIdx.x * 256 + threadIdx.x; t < M * half; t += gridDim.x * 256) {
    const int m = t / half, n = 2 * (t - m * half);
    float a = 0.f, b = 0.f;
    for (int z = 0; z < splits; ++z) {
      const float *w = p.ws + ((size_t)z * M + m) * N + n;
      a += w[0];
      b += w[1];
    }
    if (EPI == G_QKV) {
      qkv_store_pair(p.d, p.qkv, m, n, a, b);
    } else if (EPI == G_SWIGLU) {
      p.a16[(size_t)m * p.ld_a + (n >> 1)] = (_Float16)(silu(a) * b);
    } else {
      p.h[(size_t)m * p.ldh + n] += a;
      p.h[(size_t)m * p.ldh + n + 1] += b;
    }
  }
}

static dim3 grid_for(int M, int N) { return dim3((N + BN - 1) / BN, (M + BM - 1) / BM); }

// Few output tiles (small M): split K across blocks so the weight stream is
// spread over the whole chip; the partials are reduced by k_splitk_epi.
template <int EPI>
static void launch(GemmP p, const Workspace &wsp, hipStream_t st) {
  dim3 grid = grid_for(p.M, p.N);
  const int tiles = grid.x * grid.y;
  const int ksteps = p.K / BK;
  int splits = 1;
  if (EPI != G_LMHEAD && tiles < 192 && wsp.buf) {
    splits = (256 + tiles - 1) / tiles;
    splits = splits < ksteps / kStages ? splits : ksteps / kStages;
    splits = splits < 16 ? splits : 16;
    const size_t per = (size_t)p.M * p.N * 4;
    const int cap = (int)(wsp.bytes / per);
    splits = splits < cap ? splits : cap;
  }
  if (splits <= 1) {
    p.ws = nullptr;
    p.k_steps = ksteps;
    hipLaunchKernelGGL(k_gemm<EPI>, grid, dim3(256), 0, st, p);
    return;
  }
  p.k_steps = (ksteps + splits - 1) / splits;
  splits = (ksteps + p.k_steps - 1) / p.k_steps;
  p.ws = wsp.buf;
  grid.z = splits;
  hipLaunchKernelGGL(k_gemm<EPI>, grid, dim3(256), 0, st, p);
  const int pairs = p.M * (p.N / 2);
  int blocks = (pairs + 255) / 256;
  blocks = blocks < 2048 ? blocks : 2048;
  hipLaunchKernelGGL(k_splitk_epi<EPI>, dim3(blocks), dim3(256), 0, st, p, splits);
}

static GemmP base(const _Float16 *A, int lda, int M, const uint16_t *W, int N, int K) {
  GemmP p{};
  p.A = A;
  p.lda = lda;
  p.M = M;
  p.W = (const _Float16 *)W;
  p.N = N;
  p.K = K;
  return p;
}

void gemm_qkv(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
              const QkvEpi &e, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, w.wqkv, d.nqkv, d.H);
  p.d = d;
  p.qkv = e;
  launch<G_QKV>(p, ws, st);
}

void gemm_resid(const uint16_t *W, int N, int K, const _Float16 *x, int lda, int M, float *h,
                int ldh, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, W, N, K);
  p.h = h;
  p.ldh = ldh;
  launch<G_RESID>(p, ws, st);
}

void gemm_swiglu(const Dims &d, const LayerW &w, const _Float16 *x, int lda, int M,
                 _Float16 *a, int ld_a, const Workspace &ws, hipStream_t st) {
  GemmP p = base(x, lda, M, w.wgu, 2 * d.I_pad, d.H);
  p.a16 = a;
  p.ld_a = ld_a;
  launch<G_SWIGLU>(p, ws, st);
}

void gemm_lmhead(const Dims &d, const uint16_t *W, const _Float16 *x, int lda, int M,
                 const ArgmaxEpi &e, hipStream_t st) {
  GemmP p = base(x, lda, M, W, d.V, d.H);
  p.am = e;
  p.k_steps = d.H / BK;
  hipLaunchKernelGGL(k_gemm<G_LMHEAD>, grid_for(M, d.V), dim3(256), 0, st, p);
  argmax_finalize(e, M, st);
}

}  // namespace q2
