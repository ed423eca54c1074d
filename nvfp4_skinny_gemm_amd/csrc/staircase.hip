// Staircase sweep: the verify GEMM's duration as a function of the row count
// M, which is the price table StairCut cuts draft trees against (StairCut
// research page, "What it says": the check's cost rises in steps when the row
// count crosses a kernel tile boundary; release post: the staircase is
// measured, not assumed).
#include <algorithm>
#include <vector>

#include "internal.h"

using namespace nvfp4v;

namespace {

__device__ inline uint32_t mix32(uint64_t x) {
  x ^= x >> 33;
  x *= 0xff51afd7ed558ccdULL;
  x ^= x >> 33;
  x *= 0xc4ceb9fe1a85ec53ULL;
  x ^= x >> 33;
  return (uint32_t)x;
}

// Fill `copies` packed matrices with random codes and finite scales in
// [2^-3, 2^1] (bytes 0x20..0x40), so the sweep times real dequantisation.
__global__ void k_fill_packed(uint8_t *buf, size_t copy_stride, int copies, int64_t nrt,
                              int64_t nkt, uint64_t seed) {
  const size_t per = (size_t)nrt * (size_t)nkt * TILE_BYTES;
  const size_t total = per * (size_t)copies;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const size_t c = i / per, off = i - c * per;
    const size_t in_tile = off % TILE_BYTES;
    const uint32_t r = mix32(seed ^ (i * 0x9E3779B97F4A7C15ULL));
    uint8_t v = (uint8_t)r;
    if (in_tile >= (size_t)SCALE_OFFSET) v = (uint8_t)(0x20 + (r % 0x21));
    buf[c * copy_stride + off] = v;
  }
}

__global__ void k_fill_act(uint16_t *a, size_t count, uint64_t seed) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint32_t r = mix32(seed + i);
    a[i] = (uint16_t)(0x3F00u | (r & 0x00FFu) | ((r >> 8) & 0x8000u));
  }
}

}  // namespace

extern "C" int nvfp4v_staircase(nvfp4v_ctx *ctx, int64_t n, int64_t k, int m_lo, int m_hi,
                                int warmup, int reps, size_t rotate_bytes, double *us_out) {
  if (!ctx || !us_out) return NVFP4V_E_INVALID_ARG;
  if (m_lo < 1 || m_hi > NVFP4V_MAX_M || m_lo > m_hi) return NVFP4V_E_M_RANGE;
  if (reps < 1 || warmup < 0) return NVFP4V_E_INVALID_ARG;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const size_t per = L.bytes();
  const size_t stride = (per + 255) & ~size_t(255);
  size_t copies = rotate_bytes > per ? (rotate_bytes + per - 1) / per : 1;
  copies = std::min<size_t>(copies, 4096);

  uint8_t *w = nullptr;
  uint8_t *act = nullptr;
  uint16_t *a = nullptr;
  float *c = nullptr;
  hipStream_t s = nullptr;
  // Each M is timed as `reps` back-to-back launches between one pair of events,
  // repeated over `rounds` batches, and the median batch is kept: a pair of
  // events around a single launch would add the dispatch latency of a launch
  // from an idle queue (about 6 us) to the kernel's duration.
  constexpr int rounds = 5;
  std::vector<hipEvent_t> ev((size_t)rounds * 2, nullptr);
  int rc = NVFP4V_OK;
  hipError_t e = hipMalloc((void **)&w, stride * copies);
  if (e == hipSuccess) e = hipMalloc((void **)&a, (size_t)NVFP4V_MAX_M * (size_t)k * 2);
  if (e == hipSuccess) e = hipMalloc((void **)&act, act_packed_bytes(NVFP4V_MAX_M, k));
  if (e == hipSuccess) e = hipMalloc((void **)&c, (size_t)NVFP4V_MAX_M * (size_t)n * 4);
  if (e == hipSuccess) e = hipStreamCreate(&s);
  for (size_t i = 0; e == hipSuccess && i < ev.size(); ++i) e = hipEventCreate(&ev[i]);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_fill_packed, dim3(4096), dim3(256), 0, s, w, stride, (int)copies, L.nrt,
                       L.nkt, 0x5EEDULL);
    hipLaunchKernelGGL(k_fill_act, dim3(256), dim3(256), 0, s, a, (size_t)NVFP4V_MAX_M * (size_t)k,
                       0xA11CEULL);
    e = hipGetLastError();
  }
  size_t rot = 0;
  // One untimed launch on every weight copy (at most 256) before the first
  // timed M: the first launches after the fill ran 7-10 % longer than later
  // ones at the same plan (kernel durations), which made the first M of the
  // sweep look dearer than the next ones.
  if (e == hipSuccess) rc = launch_pack_rows(ctx, a, m_lo, k, act, s);
  for (size_t i = 0; e == hipSuccess && rc == NVFP4V_OK && i < std::min<size_t>(copies, 256); ++i, ++rot)
    rc = launch_gemm_rows(ctx, act, m_lo, k, w + (rot % copies) * stride, n, 1.0f, c, s);
  // Activations are packed once per M (as the chained pass does); each timed
  // launch is the GEMM alone (M > 64: one launch per block of 64 rows).
  for (int m = m_lo; e == hipSuccess && rc == NVFP4V_OK && m <= m_hi; ++m) {
    rc = launch_pack_rows(ctx, a, m, k, act, s);
    for (int i = 0; i < warmup && rc == NVFP4V_OK; ++i, ++rot)
      rc = launch_gemm_rows(ctx, act, m, k, w + (rot % copies) * stride, n, 1.0f, c, s);
    for (int b = 0; b < rounds && rc == NVFP4V_OK && e == hipSuccess; ++b) {
      e = hipEventRecord(ev[2 * b], s);
      for (int i = 0; i < reps && rc == NVFP4V_OK && e == hipSuccess; ++i, ++rot)
        rc = launch_gemm_rows(ctx, act, m, k, w + (rot % copies) * stride, n, 1.0f, c, s);
      if (e == hipSuccess && rc == NVFP4V_OK) e = hipEventRecord(ev[2 * b + 1], s);
    }
    if (e == hipSuccess && rc == NVFP4V_OK) e = hipStreamSynchronize(s);
    if (e == hipSuccess && rc == NVFP4V_OK) {
      std::vector<double> t((size_t)rounds);
      for (int b = 0; b < rounds && e == hipSuccess; ++b) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, ev[2 * b], ev[2 * b + 1]);
        t[(size_t)b] = 1000.0 * (double)ms / reps;
      }
      std::sort(t.begin(), t.end());
      us_out[m - m_lo] = t[(size_t)rounds / 2];
    }
  }
  if (e != hipSuccess && rc == NVFP4V_OK) rc = hip_status(ctx, e);
  if (s) (void)hipStreamSynchronize(s);
  for (auto &x : ev)
    if (x) (void)hipEventDestroy(x);
  if (s) (void)hipStreamDestroy(s);
  if (w) (void)hipFree(w);
  if (a) (void)hipFree(a);
  if (act) (void)hipFree(act);
  if (c) (void)hipFree(c);
  return rc;
}
