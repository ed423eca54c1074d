// NVFP4 format: quantiser (host and device), E4M3 encoding, pack / unpack
// between the canonical format and the packed device layout (internal.h).
#include <cmath>
#include <thread>
#include <vector>

#include "internal.h"

using namespace nvfp4v;

// ---------------------------------------------------------------- host -----
extern "C" int nvfp4v_quantize_host(const float *w, int64_t n, int64_t k, uint8_t *codes,
                                    uint8_t *scales) {
  if (!w || !codes || !scales) return NVFP4V_E_INVALID_ARG;
  if (n < 1 || k < 16 || k % 16 != 0) return NVFP4V_E_SHAPE;
  const int64_t total = n * k;
  for (int64_t i = 0; i < total; ++i)
    if (!std::isfinite(w[i])) return NVFP4V_E_NONFINITE;
  unsigned hw = std::thread::hardware_concurrency();
  int64_t threads = hw ? (int64_t)hw : 1;
  if (threads > 32) threads = 32;
  if (threads > n) threads = n;
  auto work = [=](int64_t t) {
    for (int64_t j = t; j < n; j += threads)
      for (int64_t b = 0; b < k / 16; ++b)
        scales[j * (k / 16) + b] =
            (uint8_t)quantize_block(w + j * k + b * 16, codes + j * (k / 2) + b * 8);
  };
  if (threads <= 1) {
    work(0);
  } else {
    std::vector<std::thread> pool;
    for (int64_t t = 0; t < threads; ++t) pool.emplace_back(work, t);
    for (auto &th : pool) th.join();
  }
  return NVFP4V_OK;
}

extern "C" int nvfp4v_encode_e4m3_host(const float *x, int64_t count, uint8_t *out) {
  if (!x || !out || count < 0) return NVFP4V_E_INVALID_ARG;
  for (int64_t i = 0; i < count; ++i)
    if (std::isnan(x[i])) return NVFP4V_E_NONFINITE;
  for (int64_t i = 0; i < count; ++i) {
    const double v = (double)x[i];
    const uint32_t mag = e4m3_encode_mag(v < 0 ? -v : v);
    out[i] = (uint8_t)(mag | (std::signbit(v) ? 0x80u : 0u));
  }
  return NVFP4V_OK;
}

extern "C" size_t nvfp4v_packed_bytes(int64_t n, int64_t k) {
  Layout L;
  if (!make_layout(n, k, &L)) return 0;
  return L.bytes();
}

// -------------------------------------------------------------- device -----
// One thread per 16-element block.
__global__ void k_quantize(const float *__restrict__ w, int64_t n, int64_t k,
                           uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const int64_t nb = k / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * nb) return;
  const int64_t j = idx / nb, b = idx - j * nb;
  float v[16];
  const float4 *src = reinterpret_cast<const float4 *>(w + j * k + b * 16);
  for (int t = 0; t < 4; ++t) {
    const float4 f = src[t];
    v[4 * t] = f.x;
    v[4 * t + 1] = f.y;
    v[4 * t + 2] = f.z;
    v[4 * t + 3] = f.w;
  }
  uint8_t c8[8];
  scales[idx] = (uint8_t)quantize_block(v, c8);
  uint2 packed;
  packed.x = (uint32_t)c8[0] | ((uint32_t)c8[1] << 8) | ((uint32_t)c8[2] << 16) | ((uint32_t)c8[3] << 24);
  packed.y = (uint32_t)c8[4] | ((uint32_t)c8[5] << 8) | ((uint32_t)c8[6] << 16) | ((uint32_t)c8[7] << 24);
  *reinterpret_cast<uint2 *>(codes + j * (k / 2) + b * 8) = packed;
}

extern "C" int nvfp4v_quantize(nvfp4v_ctx *ctx, const float *w, int64_t n, int64_t k,
                               uint8_t *codes, uint8_t *scales, hipStream_t stream) {
  if (!ctx || !w || !codes || !scales) return NVFP4V_E_INVALID_ARG;
  if (n < 1 || k < 16 || k % 16 != 0) return NVFP4V_E_SHAPE;
  if (!aligned16(w) || ((uintptr_t)codes & 7) != 0) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const int64_t blocks = n * (k / 16);
  const int threads = 256;
  const int64_t grid = (blocks + threads - 1) / threads;
  if (grid > 0x7FFFFFFF) return NVFP4V_E_SHAPE;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(threads), 0, stream, w, n, k, codes,
                     scales);
  return hip_status(ctx, hipGetLastError());
}

// Pack: one thread per (row tile, k tile, lane) writes that lane's 32 code
// bytes (two 16-byte halves) and its 4 scale bytes.
__global__ void k_pack(const uint8_t *__restrict__ codes, const uint8_t *__restrict__ scales,
                       int64_t n, int64_t k, int64_t nrt, int64_t nkt, uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nrt * nkt * 64) return;
  const int L = (int)(idx & 63);
  const int64_t tile = idx >> 6;
  const int64_t rt = tile / nkt, kt = tile - rt * nkt;
  const int r = L & 15, h = L >> 4;
  const int64_t row = rt * ROWS_PER_TILE + r;
  uint8_t *t = out + tile * (int64_t)TILE_BYTES;
  const int64_t kb = k / 2;  // code bytes per row
  for (int c = 0; c < 2; ++c) {
    uint8_t *dst = t + c * CODE_HALF_BYTES + L * 16;
    for (int i = 0; i < 16; ++i) {
      const int64_t byte = kt * 128 + h * 32 + c * 16 + i;
      dst[i] = (row < n && byte < kb) ? codes[row * kb + byte] : (uint8_t)0;
    }
  }
  const int64_t sb = k / 16;
  for (int e = 0; e < 4; ++e) {
    const int64_t blk = kt * 16 + h * 4 + e;
    t[SCALE_OFFSET + L * 4 + e] = (row < n && blk < sb) ? scales[row * sb + blk] : (uint8_t)0;
  }
}

// Unpack: the inverse gather, one thread per canonical (row, 16-block).
__global__ void k_unpack(const uint8_t *__restrict__ in, int64_t n, int64_t k, int64_t nkt,
                         uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
  const int64_t nb = k / 16;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n * nb) return;
  const int64_t row = idx / nb, blk = idx - row * nb;
  const int64_t rt = row / ROWS_PER_TILE;
  const int r = (int)(row - rt * ROWS_PER_TILE);
  const int64_t kt = blk / 16;
  const int q = (int)(blk % 16);  // 16-block within the k-tile = 4h + e
  const int h = q / 4, e = q % 4;
  const int L = r + 16 * h;
  const uint8_t *t = in + (rt * nkt + kt) * (int64_t)TILE_BYTES;
  scales[row * nb + blk] = t[SCALE_OFFSET + L * 4 + e];
  // block e of the lane's 64 k = 8 code bytes: half c = e / 2, offset 8 * (e % 2)
  const uint8_t *csrc = t + (e / 2) * CODE_HALF_BYTES + L * 16 + (e % 2) * 8;
  for (int i = 0; i < 8; ++i) codes[row * (k / 2) + blk * 8 + i] = csrc[i];
}

extern "C" int nvfp4v_pack(nvfp4v_ctx *ctx, const uint8_t *codes, const uint8_t *scales, int64_t n,
                           int64_t k, void *packed, hipStream_t stream) {
  if (!ctx || !codes || !scales || !packed) return NVFP4V_E_INVALID_ARG;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(packed)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const int64_t threads = L.nrt * L.nkt * 64;
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7FFFFFFF) return NVFP4V_E_SHAPE;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)grid), dim3(256), 0, stream, codes, scales, n, k, L.nrt,
                     L.nkt, (uint8_t *)packed);
  return hip_status(ctx, hipGetLastError());
}

extern "C" int nvfp4v_unpack(nvfp4v_ctx *ctx, const void *packed, int64_t n, int64_t k,
                             uint8_t *codes, uint8_t *scales, hipStream_t stream) {
  if (!ctx || !codes || !scales || !packed) return NVFP4V_E_INVALID_ARG;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(packed)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const int64_t threads = n * (k / 16);
  const int64_t grid = (threads + 255) / 256;
  if (grid > 0x7FFFFFFF) return NVFP4V_E_SHAPE;
  hipLaunchKernelGGL(k_unpack, dim3((unsigned)grid), dim3(256), 0, stream, (const uint8_t *)packed,
                     n, k, L.nkt, codes, scales);
  return hip_status(ctx, hipGetLastError());
}
