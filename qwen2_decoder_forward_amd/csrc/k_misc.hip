// Embedding gather, row RMSNorm and row copies.
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

// One block per row: y = w * x / sqrt(mean(x^2) + eps), stored as f16 (MFMA
// operand) and optionally f32.  When a split-K residual GEMM left `splits`
// partial sums part[z][m][k] (z < splits), they are first added to the row,
// which is written back: h[m] += sum_z part[z][m].  Thread t owns 4-float
// chunks t, t + 256, ... of the row (H <= 5120: at most 5), and issues the
// loads of its chunk of every partial at once.
__global__ __launch_bounds__(256) void k_rmsnorm_rows(float *h, int ldh, const float *w, int H,
                                                      int M, float eps, _Float16 *x, int ldx,
                                                      float *y32, const float *part, int splits) {
  constexpr int kMaxChunks = 5;  // 256 threads * 4 floats * 5 = 5120 (the supported maximum)
  __shared__ float sRed[4];
  const int m = blockIdx.x, tid = threadIdx.x;
  float *row = h + (size_t)m * ldh;
  f4 v[kMaxChunks];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int k = (tid + c * 256) * 4;
    if (k < H) {
      v[c] = *(const f4 *)(row + k);
      if (splits > 0) {
        // every partial set's load in flight at once (set index clamped,
        // the sets past `splits` masked), then the sum in set order
        f4 pz[kMaxSplits];
#pragma unroll
        for (int z = 0; z < kMaxSplits; ++z)
          pz[z] = *(const f4 *)(part + ((size_t)min(z, splits - 1) * M + m) * H + k);
#pragma unroll
        for (int z = 0; z < kMaxSplits; ++z)
          if (z < splits) v[c] += pz[z];
        *(f4 *)(row + k) = v[c];
      }
      ss += v[c].x * v[c].x + v[c].y * v[c].y + v[c].z * v[c].z + v[c].w * v[c].w;
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) sRed[tid >> 6] = ss;
  __syncthreads();
  ss = (sRed[0] + sRed[1]) + (sRed[2] + sRed[3]);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int k = (tid + c * 256) * 4;
    if (k < H) {
      const f4 g = *(const f4 *)(w + k);
      const f4 y = v[c] * inv * g;
      h4 yh = {(_Float16)y.x, (_Float16)y.y, (_Float16)y.z, (_Float16)y.w};
      *(h4 *)(x + (size_t)m * ldx + k) = yh;
      if (y32) *(f4 *)(y32 + (size_t)m * H + k) = y;
    }
  }
}

void rmsnorm_rows_f16(float *h, int ldh, const float *w, int H, int M, float eps, _Float16 *x,
                      int ldx, float *y32, const float *part, int splits, hipStream_t st) {
  hipLaunchKernelGGL(k_rmsnorm_rows, dim3(M), dim3(256), 0, st, h, ldh, w, H, M, eps, x, ldx,
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

}  // namespace q2
