// Device ceilings the measurements are set against, measured on the device
// itself in the same job as the workload: the rate at which a plain
// streaming kernel reads HBM, and the dense f16 MFMA rate of a loop that
// keeps its operands in registers.  The spec peaks (8 TB/s, 2.5 PFLOP/s)
// are not reachable in practice: HBM refresh and page switches cost read
// bandwidth, and the clock drops under sustained MFMA load.
#include <string>

#include "../../include/qwen2.h"
#include "q2_device.h"

namespace q2 {

typedef unsigned u4v __attribute__((ext_vector_type(4)));

// Every thread walks the buffer with a grid stride, 8 independent 16-byte
// non-temporal loads per step (all issued before any is used), and folds
// the words it read into one value; each wavefront's fold goes to out so
// that no load is dead.
__global__ __launch_bounds__(256) void k_probe_read(const u4v *buf, size_t n16, unsigned *out) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u4v v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u4v v = __builtin_nontemporal_load(buf + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

// Four wavefronts per block, each running `iters` rounds of four
// independent v_mfma_f32_32x32x16_f16 on register operands (values derived
// from the lane, so the operands are not constant), then storing one sum
// of its accumulators per lane group.
__global__ __launch_bounds__(256) void k_probe_mfma(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  h8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (_Float16)(0.001f * (float)((lane * 7 + j * 3) % 17) - 0.008f);
    b[j] = (_Float16)(0.001f * (float)((lane * 5 + j * 11) % 13) - 0.006f);
  }
  f16x c0, c1, c2, c3;
#pragma unroll
  for (int r = 0; r < 16; ++r) c0[r] = c1[r] = c2[r] = c3[r] = 0.f;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  s = wave_sum(s);
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace q2

namespace {
int probe_error(const char *msg) {
  q2::set_static_error(msg);
  return QWEN2_E_ARG;
}
}  // namespace

extern "C" int qwen2_probe_read(const void *buf_dev, size_t bytes, int32_t n_blocks,
                                uint32_t *out_dev, void *stream) {
  if (!buf_dev || !out_dev || bytes == 0 || bytes % 16 != 0 || n_blocks < 1 ||
      n_blocks > 65536)
    return probe_error("qwen2_probe_read: bytes must be a positive multiple of 16 and n_blocks in "
                       "[1, 65536], with non-null buffers");
  hipLaunchKernelGGL(q2::k_probe_read, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream,
                     (const q2::u4v *)buf_dev, bytes / 16, (unsigned *)out_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    q2::set_static_error(std::string("qwen2_probe_read: ") + hipGetErrorString(e));
    return QWEN2_E_HIP;
  }
  return QWEN2_OK;
}

extern "C" int qwen2_probe_mfma(int32_t iters, int32_t n_blocks, float *out_dev, void *stream) {
  if (!out_dev || iters < 1 || n_blocks < 1 || n_blocks > 65536)
    return probe_error("qwen2_probe_mfma: iters >= 1 and n_blocks in [1, 65536], with a non-null "
                       "output");
  hipLaunchKernelGGL(q2::k_probe_mfma, dim3(n_blocks), dim3(256), 0, (hipStream_t)stream, iters,
                     out_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    q2::set_static_error(std::string("qwen2_probe_mfma: ") + hipGetErrorString(e));
    return QWEN2_E_HIP;
  }
  return QWEN2_OK;
}
