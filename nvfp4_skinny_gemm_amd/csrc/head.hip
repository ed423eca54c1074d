// The FP8 output head: C[M][N] = A[M][K] * W8[N][K]^T, where W8 holds OCP E4M3
// codes with one fp32 scale per weight row, M = 1..32, on gfx950.
//
// The served model keeps every projection in NVFP4 and its output head in FP8
// (TandemLLM manual, "What TandemLLM is", 1.2 "Two levers"); the head is the
// step right after the last layer of a verify pass, over the same tree rows.
// The pages fix neither the FP8 variant nor the scale granularity; this file
// reads them as OCP E4M3 ("FN") codes and a per-row fp32 scale:
//   s(j) = fp32(absmax_k |w(j,k)| / 448),  code = E4M3_RNE(w / s) (saturating).
// A per-row scale commutes with the sum over K, so it is applied once per
// output in the epilogue and the inner loop only converts codes.
//
// Packed layout (bytes), N x K cut into 16-row x 256-k tiles like the NVFP4
// layout, one contiguous stripe per row tile:
//   tile(rt, kt) = (rt * nkt + kt) * 4096
//   load p = 0..3: bytes [1024 p + 16 L, +16), lane L = r + 16 h (r = row in
//                  tile, h = 0..3): W8[16 rt + r][256 kt + 64 h + 16 p + b]
//   after all tiles: fp32 scales[16 nrt] (rows >= N hold 0)
// so a wave reads a tile with four fully coalesced 1 KiB loads, and the 8
// bytes a lane feeds to MFMA i = 2 p + c are dwords 2c, 2c + 1 of load p: the
// same k order (64 h + 8 i + e) as the packed activations' fragment i.
//
// Kernels: the 4 waves of a work-group split N. A wave owns R row tiles over
// all of K and needs no cross-wave reduction; its weight tiles stream through
// a two-deep register ring (loads past the matrix return zeros). The
// activations reach the waves either through one copy per work-group in LDS
// (k_head_lds, the default) or through each wave's own two-deep ring of
// fragment loads (k_head). E4M3 -> bf16 is exact (4 significant bits, range
// 2^-9 .. 448): v_cvt_pk_f32_fp8 and the high halves packed with v_perm_b32.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "gemm_device.h"

using namespace nvfp4v;

namespace {

using namespace nvfp4v::dev;

constexpr int HEAD_TILE_BYTES = 4096;
constexpr int HEAD_MAX_M = NVFP4V_MAX_M;  // one launch per block of 64 rows

struct HeadArgs {
  const uint8_t *W;      // packed tiles, then the padded row scales
  const float *scales;   // W + nrt * nkt * 4096
  const uint8_t *act;    // packed activations
  float *C;              // [M][N]
  int act_bytes, M, N, nrt, nkt;
};

struct HTile {
  uint4 c[4];
};

__device__ inline void load_htile(HTile &t, __amdgpu_buffer_rsrc_t rs, int kt, bool ok, int lane) {
  const int base = ok ? kt * HEAD_TILE_BYTES : OOB;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, base + p * 1024 + lane * 16, 0, WEIGHT_AUX);
    __builtin_memcpy(&t.c[p], &x, 16);
  }
}

// Two E4M3 bytes (the low or high half of w) -> bf16x2, exact.
template <bool HI>
__device__ inline uint32_t fp8_pair(uint32_t w) {
  const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return __builtin_amdgcn_perm(__float_as_uint(v.y), __float_as_uint(v.x), 0x07060302u);
}

__device__ inline bf16x8 fp8x8(uint32_t lo, uint32_t hi) {
  uint32_t o[4] = {fp8_pair<false>(lo), fp8_pair<true>(lo), fp8_pair<false>(hi), fp8_pair<true>(hi)};
  bf16x8 r;
  __builtin_memcpy(&r, o, 16);
  return r;
}

template <int MB>
__device__ inline void compute_htile(const HTile &t, const bf16x8 (&b)[MB][8], f32x4 (&acc)[MB]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 &q = t.c[i >> 1];
    const bf16x8 wf = (i & 1) ? fp8x8(q.z, q.w) : fp8x8(q.x, q.y);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, b[mb][i], acc[mb], 0, 0, 0);
  }
}

// Three or four row blocks of activation fragments in a two-deep ring take
// most of a SIMD's registers: one wave per SIMD there.
template <int MB>
constexpr int head_waves_per_simd() {
  return MB <= 2 ? 2 : 1;
}

template <int MB, int R>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(1, head_waves_per_simd<MB>())))
void k_head(HeadArgs g) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt0 = ((int)blockIdx.x * WG_WAVES + wave) * R;
  if (rt0 >= g.nrt) return;  // wave-uniform; the kernel has no barrier
  const int stripe = g.nkt * HEAD_TILE_BYTES;
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    const uint8_t *base = g.W + (size_t)min(rt, g.nrt - 1) * (size_t)stripe;
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, rt < g.nrt ? stripe : 0,
                                              RAW_BUFFER_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.act, (short)0, g.act_bytes, RAW_BUFFER_FLAGS);

  f32x4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slot d holds k-tiles d, d + 2, ...; it is refilled two k-tiles ahead
  // right after it is consumed. A slot past the last k-tile holds zeros.
  HTile w[2][R];
  bf16x8 a[2][MB][8];
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    load_afrag<MB>(a[d], ra, d, d < g.nkt, g.M, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) load_htile(w[d][r], rs[r], d, d < g.nkt, lane);
  }
  for (int i = 0; i < g.nkt; i += 2) {
#pragma unroll
    for (int d = 0; d < 2; ++d) {
#pragma unroll
      for (int r = 0; r < R; ++r) compute_htile<MB>(w[d][r], a[d], acc[r]);
      const int nk = i + d + 2;
      load_afrag<MB>(a[d], ra, nk, nk < g.nkt, g.M, lane);
#pragma unroll
      for (int r = 0; r < R; ++r) load_htile(w[d][r], rs[r], nk, nk < g.nkt, lane);
    }
  }

  // Lane L holds rows 16 rt + 4 (L >> 4) + e (e = 0..3) of column 16 mb + (L & 15).
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    if (rt >= g.nrt) break;
    const int n0 = rt * 16 + 4 * (lane >> 4);
    const f32x4 s = *reinterpret_cast<const f32x4 *>(g.scales + n0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + (lane & 15);
      if (m >= g.M) continue;
      float *crow = g.C + (size_t)m * (size_t)g.N;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + e < g.N) crow[n0 + e] = s[e] * acc[r][mb][e];
    }
  }
}

// The same head with the activations staged in LDS once per work-group
// instead of once per wave: per k-tile every thread moves MB x 32 bytes of
// the packed activations (read two k-tiles ahead into registers, written one
// k-tile ahead into a two-slot LDS ring), and each wave reads its MFMA
// fragments from LDS. One work-group barrier per k-tile, so every wave runs
// the whole loop, also one whose row tiles lie past the matrix (its weight
// loads return zeros and it writes nothing).
template <int MB, int R>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(1, head_waves_per_simd<MB>())))
void k_head_lds(HeadArgs g) {
  constexpr int SLOT = MB * 8 * ACT_FRAG_BYTES;       // one k-tile of packed activations
  constexpr int PER_THREAD = SLOT / WG_THREADS / 16;  // 16-byte chunks per thread (2 MB)
  __shared__ __align__(16) uint8_t lds[2 * SLOT];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt0 = ((int)blockIdx.x * WG_WAVES + wave) * R;
  const int n = g.nkt;
  const int stripe = n * HEAD_TILE_BYTES;
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    const uint8_t *base = g.W + (size_t)min(rt, g.nrt - 1) * (size_t)stripe;
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, rt < g.nrt ? stripe : 0,
                                              RAW_BUFFER_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)g.act, (short)0, g.act_bytes, RAW_BUFFER_FLAGS);

  // k-tile j's packed block is contiguous (SLOT bytes at j * SLOT); thread t
  // moves chunks t, t + 256, ... of it. Rows >= M are zeros in the block.
  auto stage_load = [&](uint4 (&v)[PER_THREAD], int j) {
    const int base = j < n ? j * SLOT : OOB;
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(ra, base + (c * WG_THREADS + tid) * 16, 0, 0);
      __builtin_memcpy(&v[c], &x, 16);
    }
  };
  auto stage_store = [&](const uint4 (&v)[PER_THREAD], int slot) {
    uint4 *dst = reinterpret_cast<uint4 *>(lds + slot * SLOT);
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) dst[c * WG_THREADS + tid] = v[c];
  };
  auto frags = [&](bf16x8 (&b)[MB][8], int slot) {
    const uint4 *src = reinterpret_cast<const uint4 *>(lds + slot * SLOT);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 x = src[(mb * 8 + q) * 64 + lane];
        __builtin_memcpy(&b[mb][q], &x, 16);
      }
  };

  f32x4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  HTile w0[R], w1[R];
  uint4 s0[PER_THREAD], s1[PER_THREAD];
  stage_load(s0, 0);
#pragma unroll
  for (int r = 0; r < R; ++r) load_htile(w0[r], rs[r], 0, true, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(s1, 1);
#pragma unroll
  for (int r = 0; r < R; ++r) load_htile(w1[r], rs[r], 1, n > 1, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(s0, 0);
  stage_load(s0, 2);
  __builtin_amdgcn_sched_barrier(0);

  // Iteration i: barrier (slot i % 2 holds k-tile i, the other slot is free),
  // fragments of k-tile i, k-tile i + 1 into the free slot, k-tile i + 3's
  // activations requested, compute, then k-tile i + 2's weights requested
  // into the registers the compute has just freed.
#define NVFP4V_HEAD_STEP(W, S_NEXT, SLOT_I)                                                 \
  {                                                                                           \
    lds_barrier_wg();                                                                         \
    bf16x8 b[MB][8];                                                                          \
    frags(b, SLOT_I);                                                                         \
    stage_store(S_NEXT, 1 - SLOT_I);                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    stage_load(S_NEXT, i + 3);                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    _Pragma("unroll") for (int r = 0; r < R; ++r) compute_htile<MB>(W[r], b, acc[r]);        \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    _Pragma("unroll") for (int r = 0; r < R; ++r) load_htile(W[r], rs[r], i + 2, i + 2 < n, lane); \
    __builtin_amdgcn_sched_barrier(0);                                                        \
  }
  int i = 0;
  for (; i + 1 < n; i += 2) {
    NVFP4V_HEAD_STEP(w0, s1, 0)
    ++i;
    NVFP4V_HEAD_STEP(w1, s0, 1)
    --i;
  }
  if (i < n) NVFP4V_HEAD_STEP(w0, s1, 0)
#undef NVFP4V_HEAD_STEP

  // Lane L holds rows 16 rt + 4 (L >> 4) + e (e = 0..3) of column 16 mb + (L & 15).
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    if (rt >= g.nrt) break;
    const int n0 = rt * 16 + 4 * (lane >> 4);
    const f32x4 sc = *reinterpret_cast<const f32x4 *>(g.scales + n0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + (lane & 15);
      if (m >= g.M) continue;
      float *crow = g.C + (size_t)m * (size_t)g.N;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + e < g.N) crow[n0 + e] = sc[e] * acc[r][mb][e];
    }
  }
}

bool head_shape_ok(int64_t n, int64_t k) {
  // k <= 2^22 keeps a stripe (nkt * 4096 bytes) below 64 MiB, well inside a
  // buffer resource's 32-bit range; n <= 2^28 keeps row indices in int.
  return n >= 1 && k >= 16 && k % 16 == 0 && n <= (int64_t(1) << 28) && k <= (int64_t(1) << 22);
}

size_t head_bytes(int64_t n, int64_t k) {
  const int64_t nrt = (n + 15) / 16, nkt = (k + 255) / 256;
  return (size_t)nrt * (size_t)nkt * HEAD_TILE_BYTES + (size_t)nrt * 16 * sizeof(float);
}

typedef void (*HeadKernel)(HeadArgs);

// R row tiles per wave: 2 (measured on MI355X for 151936 x 5120 with the LDS
// stage: 121 / 134 / 154 us at M = 1 / 16 / 32, against 120 / 134 / 168 with
// R = 1 and 137 / 145 / 154 with R = 4). NVFP4V_HEAD_R=1|2|4 overrides (4 only
// at M <= 16).
int head_r(int mblocks) {
  if (const char *ov = std::getenv("NVFP4V_HEAD_R")) {
    const int r = std::atoi(ov);
    if (r == 1 || r == 2 || (r == 4 && mblocks == 1)) return r;
  }
  return 2;
}

HeadKernel pick_head(int mblocks, int r) {
  switch (mblocks) {
    case 1: return r == 1 ? k_head<1, 1> : r == 2 ? k_head<1, 2> : k_head<1, 4>;
    case 2: return r == 1 ? k_head<2, 1> : k_head<2, 2>;
    case 3: return r == 1 ? k_head<3, 1> : k_head<3, 2>;
    default: return r == 1 ? k_head<4, 1> : k_head<4, 2>;
  }
}

HeadKernel pick_head_lds(int mblocks, int r) {
  switch (mblocks) {
    case 1: return r == 1 ? k_head_lds<1, 1> : r == 2 ? k_head_lds<1, 2> : k_head_lds<1, 4>;
    case 2: return r == 1 ? k_head_lds<2, 1> : k_head_lds<2, 2>;
    case 3: return r == 1 ? k_head_lds<3, 1> : k_head_lds<3, 2>;
    default: return r == 1 ? k_head_lds<4, 1> : k_head_lds<4, 2>;
  }
}

// Activations staged in LDS per work-group (k_head_lds) or loaded per wave
// (k_head): LDS at every M, measured on MI355X for 151936 x 5120 at R = 2
// (121 / 134 / 142 / 154 / 198 / 239 us at M = 1 / 16 / 17 / 32 / 48 / 64,
// against 122 / 144 / 165 / 191 / 243 / 279 with per-wave loads).
// NVFP4V_HEAD_LDS=0|1 overrides.
bool head_lds() {
  if (const char *ov = std::getenv("NVFP4V_HEAD_LDS")) return std::atoi(ov) != 0;
  return true;
}

// One launch over a block of at most 64 rows (m <= CHUNK_M).
int launch_head_block(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                      int64_t n, float *c, hipStream_t stream) {
  HeadArgs g;
  g.nrt = (int)((n + 15) / 16);
  g.nkt = (int)((k + 255) / 256);
  g.W = (const uint8_t *)packed;
  g.scales = (const float *)(g.W + (size_t)g.nrt * (size_t)g.nkt * HEAD_TILE_BYTES);
  g.act = act;
  g.act_bytes = (int)act_copy_bytes(m, k);
  g.C = c;
  g.M = (int)m;
  g.N = (int)n;
  const int mblocks = (int)((m + 15) / 16);
  const int r = head_r(mblocks);
  const int rows_per_wg = WG_WAVES * r;
  const int grid = (g.nrt + rows_per_wg - 1) / rows_per_wg;
  const HeadKernel kern = head_lds() ? pick_head_lds(mblocks, r) : pick_head(mblocks, r);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WG_THREADS), 0, stream, g);
  return hip_status(ctx, hipGetLastError());
}

// Any m: one launch per block of 64 rows of the packed activations.
int launch_head(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                int64_t n, float *c, hipStream_t stream) {
  int rc = NVFP4V_OK;
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    rc = launch_head_block(ctx, act, mc, k, packed, n, c + r0 * n, stream);
    act += act_block_bytes(mc, k);
  }
  return rc;
}

int head_checks(nvfp4v_ctx *ctx, const void *a, int64_t m, int64_t k, const void *packed, int64_t n,
                const float *c) {
  if (!ctx || !a || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > HEAD_MAX_M) return NVFP4V_E_M_RANGE;
  if (!head_shape_ok(n, k)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  return NVFP4V_OK;
}

}  // namespace

extern "C" size_t nvfp4v_fp8_packed_bytes(int64_t n, int64_t k) {
  return head_shape_ok(n, k) ? head_bytes(n, k) : 0;
}

extern "C" int nvfp4v_fp8_quantize_host(const float *w, int64_t n, int64_t k, uint8_t *codes,
                                        float *row_scales) {
  if (!w || !codes || !row_scales) return NVFP4V_E_INVALID_ARG;
  if (!head_shape_ok(n, k)) return NVFP4V_E_SHAPE;
  for (int64_t i = 0; i < n * k; ++i)
    if (!std::isfinite(w[i])) return NVFP4V_E_NONFINITE;
  unsigned hw = std::thread::hardware_concurrency();
  int64_t threads = hw ? (int64_t)hw : 1;
  if (threads > 32) threads = 32;
  if (threads > n) threads = n;
  auto work = [=](int64_t t) {
    for (int64_t j = t; j < n; j += threads) {
      const float *wr = w + j * k;
      double amax = 0.0;
      for (int64_t kk = 0; kk < k; ++kk) amax = std::max(amax, std::fabs((double)wr[kk]));
      const float s = (float)(amax / 448.0);
      row_scales[j] = s;
      for (int64_t kk = 0; kk < k; ++kk) {
        if (s == 0.0f) {
          codes[j * k + kk] = 0;
          continue;
        }
        const double q = (double)wr[kk] / (double)s;
        codes[j * k + kk] = (uint8_t)(e4m3_encode_mag(std::fabs(q)) | (std::signbit(q) ? 0x80u : 0u));
      }
    }
  };
  std::vector<std::thread> pool;
  for (int64_t t = 0; t < threads; ++t) pool.emplace_back(work, t);
  for (auto &th : pool) th.join();
  return NVFP4V_OK;
}

extern "C" int nvfp4v_fp8_pack_host(const uint8_t *codes, const float *row_scales, int64_t n,
                                    int64_t k, void *packed) {
  if (!codes || !row_scales || !packed) return NVFP4V_E_INVALID_ARG;
  if (!head_shape_ok(n, k)) return NVFP4V_E_SHAPE;
  const int64_t nrt = (n + 15) / 16, nkt = (k + 255) / 256;
  uint8_t *out = (uint8_t *)packed;
  std::memset(out, 0, head_bytes(n, k));
  for (int64_t j = 0; j < n; ++j) {
    const int64_t rt = j >> 4, r = j & 15;
    for (int64_t k0 = 0; k0 < k; k0 += 16) {  // one 16-byte chunk: fixed kt, h, p
      const int64_t kt = k0 >> 8, h = (k0 >> 6) & 3, p = (k0 >> 4) & 3;
      const size_t off = (size_t)(rt * nkt + kt) * HEAD_TILE_BYTES + (size_t)(p * 1024 + (r + 16 * h) * 16);
      std::memcpy(out + off, codes + j * k + k0, 16);
    }
  }
  float *sc = (float *)(out + (size_t)nrt * (size_t)nkt * HEAD_TILE_BYTES);
  for (int64_t j = 0; j < n; ++j) sc[j] = row_scales[j];
  return NVFP4V_OK;
}

extern "C" int nvfp4v_fp8_head_gemm_pa(nvfp4v_ctx *ctx, const void *act, int64_t m, int64_t k,
                                       const void *packed, int64_t n, float *c, hipStream_t stream) {
  int rc = head_checks(ctx, act, m, k, packed, n, c);
  if (rc) return rc;
  if (fault_injected()) return NVFP4V_E_FAULT;
  return launch_head(ctx, (const uint8_t *)act, m, k, packed, n, c, stream);
}

extern "C" int nvfp4v_fp8_head_gemm(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k,
                                    const void *packed, int64_t n, float *c, hipStream_t stream) {
  int rc = head_checks(ctx, a, m, k, packed, n, c);
  if (rc) return rc;
  if (act_block_bytes(std::min<int64_t>(m, CHUNK_M), k) > ctx->act_bytes) return NVFP4V_E_WORKSPACE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    rc = launch_pack_act(ctx, a + r0 * k, mc, k, ctx->act, 0, stream);  // the bf16 copy only
    if (!rc) rc = launch_head_block(ctx, ctx->act, mc, k, packed, n, c + r0 * n, stream);
  }
  return rc;
}
