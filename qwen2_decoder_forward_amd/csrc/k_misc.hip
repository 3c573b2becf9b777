// Embedding gather, row RMSNorm, row copies, the greedy read-out's index and
// stop-id latch, and the next-token distribution (also its context-free,
// allocation-free entry point qwen2_next_token_probs_static).
#include <mutex>

#include "../../include/qwen2.h"
#include "q2_device.h"

namespace q2 {

// h[m] = f32(E[tokens[m]]): the embedding output enters the first layer
// unscaled.  An id outside [0, V) cannot be rejected on the host when the
// tokens live on the device; it reads row 0 and latches *bad.
__global__ __launch_bounds__(256) void k_embed(const uint16_t *E, int H, int V,
                                               const int *const *tokens, int tok_off, float *h,
                                               unsigned int *bad) {
  const int m = blockIdx.x;
  int t = (*tokens)[tok_off + m];
  if (t < 0 || t >= V) {
    if (threadIdx.x == 0) *bad = 1u;
    t = 0;
  }
  const _Float16 *row = (const _Float16 *)E + (size_t)t * H;
  for (int k = threadIdx.x * 8; k < H; k += 256 * 8) {
    const h8 v = *(const h8 *)(row + k);
    f4 a = {(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    f4 b = {(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
    *(f4 *)(h + (size_t)m * H + k) = a;
    *(f4 *)(h + (size_t)m * H + k + 4) = b;
  }
}

void embed_rows(const uint16_t *E, int H, int V, const int *const *tokens, int tok_off, int M,
                float *h, unsigned int *bad_flag, hipStream_t st) {
  hipLaunchKernelGGL(k_embed, dim3(M), dim3(256), 0, st, E, H, V, tokens, tok_off, h, bad_flag);
}

// One wavefront per row, four rows per block: y = w * x / sqrt(mean(x^2) +
// eps), stored as f16 (MFMA operand) and optionally f32.  When a split-K
// residual GEMM left `splits` partial sums part[z][m][k] (z < splits), they
// are first added to the row, which is written back: h[m] += sum_z
// part[z][m].  Lane l owns the 4-float chunks l, l + 64, ... of the row (H
// <= 8192: at most 32); every load of the lane (row chunks, norm gains,
// partials) is issued before the first is used, and the row's sum of
// squares is one wave reduction (no barrier).  x (f16) may be null when
// only the f32 copy is wanted.
template <int NCH>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(float *h, int ldh, const float *w, int H,
                                                      int M, float eps, _Float16 *x, int ldx,
                                                      float *y32, const float *part, int splits) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;  // (uniform across the wavefront)
  float *row = h + (size_t)m * ldh;
  f4 v[NCH], g[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int k = min((lane + c * 64) * 4, H - 4);  // (chunks past H re-read the last, unused)
    v[c] = *(const f4 *)(row + k);
    g[c] = *(const f4 *)(w + k);
  }
  if (splits > 0) {
    // two partial sets per round trip (one for the widest rows, whose
    // chunks fill the registers), summed in set order
    constexpr int ZB = NCH <= 14 ? 2 : 1;
    for (int z = 0; z < splits; z += ZB) {
      f4 pz[ZB][NCH];
#pragma unroll
      for (int u = 0; u < ZB; ++u) {
        const float *pr = part + ((size_t)min(z + u, splits - 1) * M + m) * H;
#pragma unroll
        for (int c = 0; c < NCH; ++c) pz[u][c] = *(const f4 *)(pr + min((lane + c * 64) * 4, H - 4));
      }
#pragma unroll
      for (int u = 0; u < ZB; ++u)
        if (z + u < splits)
#pragma unroll
          for (int c = 0; c < NCH; ++c) v[c] += pz[u][c];
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int k = (lane + c * 64) * 4;
      if (k < H) *(f4 *)(row + k) = v[c];
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    if ((lane + c * 64) * 4 < H) ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)H + eps);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int k = (lane + c * 64) * 4;
    if (k < H) {
      const f4 y = v[c] * inv * g[c];
      if (x) {
        h4 yh = {(_Float16)y.x, (_Float16)y.y, (_Float16)y.z, (_Float16)y.w};
        *(h4 *)(x + (size_t)m * ldx + k) = yh;
      }
      if (y32) *(f4 *)(y32 + (size_t)m * H + k) = y;
    }
  }
}

void rmsnorm_rows_f16(float *h, int ldh, const float *w, int H, int M, float eps, _Float16 *x,
                      int ldx, float *y32, const float *part, int splits, hipStream_t st) {
  const dim3 grid((M + 3) / 4);
  const int nch = (H + 255) / 256;  // 4-float chunks per lane
  if (nch <= 4)
    hipLaunchKernelGGL(k_rmsnorm_rows<4>, grid, dim3(256), 0, st, h, ldh, w, H, M, eps, x, ldx,
                       y32, part, splits);
  else if (nch <= 8)
    hipLaunchKernelGGL(k_rmsnorm_rows<8>, grid, dim3(256), 0, st, h, ldh, w, H, M, eps, x, ldx,
                       y32, part, splits);
  else if (nch <= 14)
    hipLaunchKernelGGL(k_rmsnorm_rows<14>, grid, dim3(256), 0, st, h, ldh, w, H, M, eps, x, ldx,
                       y32, part, splits);
  else
    hipLaunchKernelGGL(k_rmsnorm_rows<32>, grid, dim3(256), 0, st, h, ldh, w, H, M, eps, x, ldx,
                       y32, part, splits);
}

// dst[dst_rows[i]] = src[src_rows[i]] for i < k, ncols floats per row
// (ncols a multiple of 4, row strides multiples of 4): one block per pair.
__global__ __launch_bounds__(256) void k_copy_rows(const float *src, int lds, const int *src_rows,
                                                   float *dst, int ldd, const int *dst_rows,
                                                   int ncols) {
  const float *s = src + (size_t)src_rows[blockIdx.x] * lds;
  float *o = dst + (size_t)dst_rows[blockIdx.x] * ldd;
  for (int k = threadIdx.x * 4; k < ncols; k += 256 * 4) *(f4 *)(o + k) = *(const f4 *)(s + k);
}

void copy_rows(const float *src, int lds, const int *src_rows, float *dst, int ldd,
               const int *dst_rows, int k, int ncols, hipStream_t st) {
  if (k <= 0) return;
  hipLaunchKernelGGL(k_copy_rows, dim3(k), dim3(256), 0, st, src, lds, src_rows, dst, ldd,
                     dst_rows, ncols);
}

// The greedy result: index of each row's packed maximum, which is then
// cleared for the next call.  Runs after the lm_head kernel (the kernel
// boundary orders its atomics before these reads).  When the id is one of
// the stop ids, the row's sequence slot keeps the smallest such read-out
// position.
__global__ void k_argmax_finalize(ArgmaxEpi e, int M) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m < M) {
    const unsigned long long b = e.best[m];
    e.best[m] = 0ull;
    const int id = argmax_index(b);
    int *o = *e.out;
    if (o) o[m] = id;
    const int n_stop = e.stop[0];
    for (int i = 0; i < n_stop; ++i)
      if (id == e.stop[1 + i]) {
        atomicMin(e.stop_pos + e.rows.seq[m], (unsigned)e.rows.pos[m]);
        break;
      }
  }
}

void argmax_finalize(const ArgmaxEpi &e, int M, hipStream_t st) {
  hipLaunchKernelGGL(k_argmax_finalize, dim3((M + 255) / 256), dim3(256), 0, st, e, M);
}

// out[s] = latched stop position of slot s (-1: none); with `clear` the
// latch is reset.
__global__ void k_read_stops(unsigned *stop_pos, int n, int *out, int clear) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < n) {
    out[s] = (int)stop_pos[s];  // (~0u reads as -1)
    if (clear) stop_pos[s] = ~0u;
  }
}

void read_stops(unsigned *stop_pos, int n, int *out, int clear, hipStream_t st) {
  hipLaunchKernelGGL(k_read_stops, dim3((n + 255) / 256), dim3(256), 0, st, stop_pos, n, out,
                     clear);
}

// Next-token distribution p = softmax(logits row), in two launches over nb
// blocks per row (nb <= kProbBlocks: one per CU for a single row, fewer
// per row as rows are added, so that blocks stay busy).  First: each
// block's maximum m_b and s_b = sum over its columns of e^(x - m_b), as an
// online (max, sum) per thread, then combined over the block.
__device__ __forceinline__ void ms_combine(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == kNegInf) return;  // (both empty)
  s = s * expf(m - mm) + s2 * expf(m2 - mm);
  m = mm;
}

__global__ __launch_bounds__(256) void k_softmax_part(const float *logits, int V, float2 *part) {
  const int b = blockIdx.x, row = blockIdx.y;
  const int chunk = (V + gridDim.x - 1) / gridDim.x;
  const int c0 = b * chunk, c1 = min(V, c0 + chunk);
  const float *x = logits + (size_t)row * V;
  float m = kNegInf, s = 0.f;
  for (int i = c0 + (int)threadIdx.x; i < c1; i += 256) {
    const float v = x[i];
    if (v > m) {
      s = s * expf(m - v) + 1.f;
      m = v;
    } else {
      s += expf(v - m);
    }
  }
  // combine over the wavefront, then over the 4 wavefronts
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    ms_combine(m, s, m2, s2);
  }
  __shared__ float2 sw[4];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sw[w] = make_float2(m, s);
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 4; ++i) ms_combine(m, s, sw[i].x, sw[i].y);
    part[(size_t)row * gridDim.x + b] = make_float2(m, s);
  }
}

// Second: every block combines its row's kProbBlocks partials (one per
// thread) into the row maximum M and S = sum of e^(x - M), and writes
// e^(x - M) / S for its columns.
__global__ __launch_bounds__(256) void k_softmax_norm(const float *logits, int V,
                                                      const float2 *part, float *probs) {
  const int b = blockIdx.x, row = blockIdx.y;
  __shared__ float2 sw[4];
  {
    float m = kNegInf, s = 0.f;  // (threads past nb hold an empty partial)
    if (threadIdx.x < gridDim.x) {
      const float2 q = part[(size_t)row * gridDim.x + threadIdx.x];
      m = q.x;
      s = q.y;
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      ms_combine(m, s, m2, s2);
    }
    if ((threadIdx.x & 63) == 0) sw[threadIdx.x >> 6] = make_float2(m, s);
  }
  __syncthreads();
  float M = sw[0].x, S = sw[0].y;
  for (int i = 1; i < 4; ++i) ms_combine(M, S, sw[i].x, sw[i].y);
  const float inv = 1.0f / S;
  const int chunk = (V + gridDim.x - 1) / gridDim.x;
  const int c0 = b * chunk, c1 = min(V, c0 + chunk);
  const float *x = logits + (size_t)row * V;
  float *y = probs + (size_t)row * V;
  for (int i = c0 + (int)threadIdx.x; i < c1; i += 256) y[i] = expf(x[i] - M) * inv;
}

int softmax_blocks(int rows) { return std::max(16, std::min(kProbBlocks, 1024 / rows)); }

void softmax_rows(const float *logits, int rows, int V, float2 *part, float *probs,
                  hipStream_t st) {
  static_assert(kProbBlocks == 256, "at most one partial per thread of the combining block");
  const int nb = softmax_blocks(rows);
  const dim3 grid(nb, rows);
  hipLaunchKernelGGL(k_softmax_part, grid, dim3(256), 0, st, logits, V, part);
  hipLaunchKernelGGL(k_softmax_norm, grid, dim3(256), 0, st, logits, V, part, probs);
}

// Interleaved-RoPE models hold K with dimension 2j at j and 2j+1 at j + hd/2.
// to_pairs: natural [rows, hd] -> that order; else back.  One thread per
// (row, j).
__global__ void k_pair_order(const float *src, float *dst, int rows, int hd, int to_pairs) {
  const int half = hd / 2;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < rows * half) {
    const int r = i / half, j = i - r * half;
    const float *s = src + (size_t)r * hd;
    float *o = dst + (size_t)r * hd;
    if (to_pairs) {
      o[j] = s[2 * j];
      o[j + half] = s[2 * j + 1];
    } else {
      o[2 * j] = s[j];
      o[2 * j + 1] = s[j + half];
    }
  }
}

void pair_order(const float *src, float *dst, int rows, int hd, bool to_pairs, hipStream_t st) {
  const int n = rows * (hd / 2);
  hipLaunchKernelGGL(k_pair_order, dim3((n + 255) / 256), dim3(256), 0, st, src, dst, rows, hd,
                     (int)to_pairs);
}

}  // namespace q2

// ------------------------------------------- next_token_probs with no allocation
// The softmax partials of qwen2_next_token_probs_static live in this
// file-scope device array (one copy per GPU, kept until the process ends)
// instead of a context's scratch.  Host code never passes the array's name
// to a kernel: on the host it is only a stand-in for the symbol.  Its device
// address is looked up once per device, with that device current, and kept.
namespace {
constexpr int kStaticProbRows = 64;
constexpr int kStaticPartials = 1024;  // >= rows * softmax_blocks(rows) for rows <= 64
constexpr int kMaxDevices = 64;
static __device__ __align__(256) float2 scratch[kStaticPartials];
std::mutex g_scratch_mu;
float2 *g_scratch_ptr[kMaxDevices] = {};

int scratch_on(int dev, float2 **out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    float2 *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      q2::set_static_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return QWEN2_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QWEN2_OK;
}
}  // namespace

extern "C" int qwen2_next_token_probs_static(const float *logits_dev, int32_t rows,
                                             int32_t n_vocab, float *probs_dev, void *stream) {
  static_assert(kStaticProbRows * 16 <= kStaticPartials, "rows * blocks per row fit");
  if (!logits_dev || !probs_dev) {
    q2::set_static_error("null logits or probs");
    return QWEN2_E_ARG;
  }
  if (rows < 1 || rows > kStaticProbRows || n_vocab < 1) {
    q2::set_static_error("rows must be in [1, 64] and n_vocab >= 1");
    return QWEN2_E_ARG;
  }
  if (rows * q2::softmax_blocks(rows) > kStaticPartials) {  // (never, by the block count's rule)
    q2::set_static_error("softmax partials exceed the static scratch");
    return QWEN2_E_ARG;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    q2::set_static_error(std::string("hipGetDevice: ") + hipGetErrorString(e));
    return QWEN2_E_HIP;
  }
  float2 *part = nullptr;
  const int rc = scratch_on(dev, &part);
  if (rc) return rc;
  q2::softmax_rows(logits_dev, rows, n_vocab, part, probs_dev, (hipStream_t)stream);
  e = hipGetLastError();
  if (e != hipSuccess) {
    q2::set_static_error(std::string("softmax launch: ") + hipGetErrorString(e));
    return QWEN2_E_HIP;
  }
  return QWEN2_OK;
}
