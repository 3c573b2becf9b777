// Debug checks (a context loaded with QWEN2_DEBUG_CHECKS=1): a hash of every
// KV-cache word outside the slots a call may write, taken before and after
// the call, and scans for non-finite values in what the call wrote.  Failed
// guards are reported with the offending value; nothing here runs unless the
// context asked for it.
#include "q2_device.h"

namespace q2 {

namespace {

// Position and sequence slot of 32-bit word w of one of the cache arrays:
//  0: f32 K or V, [L][n_seq][nkv][n_ctx][hd] floats;
//  1: binary16 K mirror, [L][n_seq][nkv][ldp][hd] halves (hd / 2 words per position);
//  2: binary16 V^T mirror, [L][n_seq][nkv][hd][ldp] halves (two positions per word).
// Sets p1 to the word's second position (mode 2) or to p0.
__device__ __forceinline__ void word_slot(int mode, size_t w, const DebugKv &a, int &seq, int &p0,
                                          int &p1) {
  if (mode == 0) {
    const size_t slot = w / a.hd;
    p0 = (int)(slot % a.n_ctx);
    seq = (int)((slot / ((size_t)a.n_ctx * a.nkv)) % a.n_seq);
    p1 = p0;
  } else if (mode == 1) {
    const size_t slot = w / (a.hd / 2);
    p0 = (int)(slot % a.ldp);
    seq = (int)((slot / ((size_t)a.ldp * a.nkv)) % a.n_seq);
    p1 = p0;
  } else {
    const size_t half_row = a.ldp / 2;
    p0 = (int)(2 * (w % half_row));
    seq = (int)((w / (half_row * a.hd * a.nkv)) % a.n_seq);
    p1 = p0 + 1;
  }
}

}  // namespace

// Sums a mix of (word, index) over the words whose slots the call may not
// write (an order-free sum, so wavefronts add their shares atomically), and
// for the f32 words of slots it did write, keeps the smallest index of a
// non-finite value (~0: none).
__global__ __launch_bounds__(256) void k_debug_kv(DebugKv a, int mode, const uint32_t *words,
                                                  size_t n_words, unsigned long long salt,
                                                  unsigned long long *hash,
                                                  unsigned long long *bad) {
  unsigned long long h = 0, first_bad = ~0ull;
  for (size_t w = (size_t)blockIdx.x * 256 + threadIdx.x; w < n_words;
       w += (size_t)gridDim.x * 256) {
    int seq, p0, p1;
    word_slot(mode, w, a, seq, p0, p1);
    const bool written = (p0 < a.n_ctx && a.mask[(size_t)seq * a.n_ctx + p0]) ||
                         (p1 < a.n_ctx && a.mask[(size_t)seq * a.n_ctx + p1]);
    const uint32_t x = words[w];
    if (!written) {
      h += ((unsigned long long)x ^ ((unsigned long long)w << 32) ^ salt) * 0x9E3779B97F4A7C15ull;
    } else if (mode == 0 && (x & 0x7F800000u) == 0x7F800000u) {
      first_bad = min(first_bad, (unsigned long long)w);
    }
  }
  for (int o = 32; o >= 1; o >>= 1) {  // one atomic per wavefront
    h += shfl_xor_u64(h, o);
    first_bad = min(first_bad, shfl_xor_u64(first_bad, o));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicAdd(hash, h);
    if (first_bad != ~0ull) atomicMin(bad, first_bad);
  }
}

// Smallest index of a non-finite value among x[0 .. n).
__global__ __launch_bounds__(256) void k_debug_nonfinite(const float *x, size_t n,
                                                         unsigned long long *bad) {
  unsigned long long first_bad = ~0ull;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    if (!isfinite(x[i])) first_bad = min(first_bad, (unsigned long long)i);
  if (first_bad != ~0ull) atomicMin(bad, first_bad);
}

void debug_kv(const DebugKv &a, const float *k, const float *v, const _Float16 *k16,
              const _Float16 *v16t, size_t f32_words, size_t f16_words,
              unsigned long long *hash, unsigned long long *bad_k, unsigned long long *bad_v,
              hipStream_t st) {
  const dim3 g(1024), b(256);
  hipLaunchKernelGGL(k_debug_kv, g, b, 0, st, a, 0, (const uint32_t *)k, f32_words, 1ull, hash,
                     bad_k);
  hipLaunchKernelGGL(k_debug_kv, g, b, 0, st, a, 0, (const uint32_t *)v, f32_words, 2ull, hash,
                     bad_v);
  hipLaunchKernelGGL(k_debug_kv, g, b, 0, st, a, 1, (const uint32_t *)k16, f16_words, 3ull, hash,
                     bad_k);
  hipLaunchKernelGGL(k_debug_kv, g, b, 0, st, a, 2, (const uint32_t *)v16t, f16_words, 4ull,
                     hash, bad_v);
}

void debug_nonfinite(const float *x, size_t n, unsigned long long *bad, hipStream_t st) {
  hipLaunchKernelGGL(k_debug_nonfinite, dim3(1024), dim3(256), 0, st, x, n, bad);
}

}  // namespace q2
