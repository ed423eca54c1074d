// Measurement kernels: a read-only HBM stream (the practical read ceiling the
// verify GEMM is compared with) and a plain copy of known size (used to
// calibrate hardware byte counters).
#include "internal.h"

using namespace nvfp4v;

namespace {

constexpr int PROBE_THREADS = 256;

// Each thread reads 16-byte words strided by the whole grid, 2 loads in flight,
// and folds them with xor; one word per work-group is written so the loads
// cannot be removed. Three work-groups per CU with two 16-byte loads per lane
// in flight measured fastest on MI355X among 1..8 work-groups per CU and
// 1..16 loads per lane (more bytes in flight only adds queueing).
constexpr int PROBE_WGS_PER_CU = 3;
__global__ __launch_bounds__(PROBE_THREADS) void k_read_probe(const uint4 *__restrict__ src,
                                                              size_t words, uint32_t *sink) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  uint32_t acc = 0;
  for (; i + stride < words; i += 2 * stride) {
    const uint4 v0 = src[i], v1 = src[i + stride];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
  }
  for (; i < words; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[PROBE_THREADS];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
    for (int t = 0; t < PROBE_THREADS; ++t) a ^= red[t];
    sink[blockIdx.x] = a;
  }
}

__global__ __launch_bounds__(PROBE_THREADS) void k_copy_probe(const uint4 *__restrict__ src,
                                                              uint4 *__restrict__ dst,
                                                              size_t words) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  for (size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x; i < words; i += stride)
    dst[i] = src[i];
}

}  // namespace

extern "C" size_t nvfp4v_read_probe_sink_words(nvfp4v_ctx *ctx) {
  return ctx ? (size_t)ctx->num_cus * PROBE_WGS_PER_CU : 0;
}

extern "C" int nvfp4v_read_probe(nvfp4v_ctx *ctx, const void *buf, size_t bytes, uint32_t *sink,
                                 hipStream_t stream) {
  if (!ctx || !buf || !sink) return NVFP4V_E_INVALID_ARG;
  if (bytes == 0 || bytes % 16 != 0) return NVFP4V_E_SHAPE;
  if (!aligned16(buf)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const unsigned grid = (unsigned)(ctx->num_cus * PROBE_WGS_PER_CU);
  hipLaunchKernelGGL(k_read_probe, dim3(grid), dim3(PROBE_THREADS), 0, stream,
                     (const uint4 *)buf, bytes / 16, sink);
  return hip_status(ctx, hipGetLastError());
}

extern "C" int nvfp4v_copy_probe(nvfp4v_ctx *ctx, const void *src, void *dst, size_t bytes,
                                 hipStream_t stream) {
  if (!ctx || !src || !dst) return NVFP4V_E_INVALID_ARG;
  if (bytes == 0 || bytes % 16 != 0) return NVFP4V_E_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const unsigned grid = (unsigned)(ctx->num_cus * 8);
  hipLaunchKernelGGL(k_copy_probe, dim3(grid), dim3(PROBE_THREADS), 0, stream,
                     (const uint4 *)src, (uint4 *)dst, bytes / 16);
  return hip_status(ctx, hipGetLastError());
}
