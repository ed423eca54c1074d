// The verify GEMM: C[M][N] = ts * A[M][K] * W[N][K]^T with W in the packed
// NVFP4 layout and A in packed (MFMA fragment) order (internal.h), M = 1..64,
// on gfx950.
//
// The pass is bound by streaming the 4-bit weights from HBM (TandemLLM manual,
// "What TandemLLM is", 1.2 "Two levers": a verify pass over 16 rows reads the
// same weights as one over a single row), so the kernel is organised around
// keeping weight bytes in flight and everything else off the memory pipe:
//
//  * A work-group of 4 waves owns R row tiles (16 R weight rows) and one split
//    of the k-tiles; its waves cut the split into 4 contiguous k-ranges. A wave
//    walks its k-range; per k-tile it loads the activation fragments once
//    (one coalesced 16-byte load per lane per fragment) and reuses them for
//    all R row tiles, whose weight tiles stream through an R-deep register
//    ring: after a row tile's k-tile is consumed, the same registers are
//    refilled with that row tile's next k-tile, so about R tiles (R * 2304
//    bytes per wave) are in flight while the wave computes.
//  * Every load is an unconditional raw buffer load: a k-tile past the wave's
//    range, a row tile past N or an activation row >= M gets an offset past the
//    buffer's size, which returns zeros without a memory access. Straight-line
//    loads keep the compiler's wait counts exact.
//  * Dequantisation is exact: v_cvt_scalef32_pk_f32_fp4 turns two E2M1 codes
//    into fp32 (with a unit scale; on gfx950 the instruction applies only the
//    exponent of its scale operand), a fp32 multiply applies the E4M3 block
//    scale (v_cvt_f32_fp8 decodes it), and the high halves are packed as bf16
//    (an E2M1 value times an E4M3 scale has at most 6 significant bits and lies
//    in [2^-10, 2688]).
//  * v_mfma_f32_16x16x32_bf16 with the weights as the 16-row A operand and a
//    16-row block of activations as the B operand, fp32 accumulation.
//  * The 4 waves' tiles are summed through LDS in wave order. With ksplit > 1
//    every work-group stores its partial tile with system-coherent stores
//    (they bypass the non-coherent L2s of the other dies, so no L2 write-back
//    fence is needed), waits for them, and takes an arrival ticket; the last
//    work-group to arrive sums the partials in split order 0..ksplit-1. Both
//    orders are fixed, so C is bitwise reproducible (TandemLLM manual, 1.7 "The
//    paper": the 4-bit kernels keep a fixed reduction order). No float atomics.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include <hip/hip_bf16.h>

#include "internal.h"

using namespace nvfp4v;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WG_WAVES = 4;
constexpr int WG_THREADS = 64 * WG_WAVES;
constexpr int OOB = 0x7FFFFFF0;  // a buffer offset past every range: the load returns zeros
constexpr int RAW_BUFFER_FLAGS = 0x00020000;

template <int SEL>
__device__ inline uint32_t dq_pair(uint32_t codes, float s) {
  // Two E2M1 codes of byte SEL (low nibble = even k) -> fp32, times the block
  // scale, high halves packed as bf16x2 (exact).
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, SEL);
  const float x = v.x * s, y = v.y * s;
  return __builtin_amdgcn_perm(__float_as_uint(y), __float_as_uint(x), 0x07060302u);
}

__device__ inline bf16x8 dequant8(uint32_t codes, float s) {
  uint32_t o[4];
  o[0] = dq_pair<0>(codes, s);
  o[1] = dq_pair<1>(codes, s);
  o[2] = dq_pair<2>(codes, s);
  o[3] = dq_pair<3>(codes, s);
  bf16x8 r;
  __builtin_memcpy(&r, o, 16);
  return r;
}

// The four E4M3 scale bytes of a lane -> fp32 (OCP E4M3 on gfx950, exact).
__device__ inline void scales4(uint32_t sw, float s[4]) {
  s[0] = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
  s[1] = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
  s[2] = __builtin_amdgcn_cvt_f32_fp8((int)sw, 2);
  s[3] = __builtin_amdgcn_cvt_f32_fp8((int)sw, 3);
}

struct WTile {
  uint4 c[2];  // code halves
  uint32_t s;  // 4 scale bytes
};

// One row tile's k-tile (three loads per lane); `ok` false gives zeros.
__device__ inline void load_wtile(WTile &t, __amdgpu_buffer_rsrc_t rs, int kt, bool ok, int lane) {
  const int base = ok ? kt * TILE_BYTES : OOB;
  const auto c0 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + lane * 16, 0, 0);
  const auto c1 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + CODE_HALF_BYTES + lane * 16, 0, 0);
  const auto sc = __builtin_amdgcn_raw_buffer_load_b32(rs, base + SCALE_OFFSET + lane * 4, 0, 0);
  __builtin_memcpy(&t.c[0], &c0, 16);
  __builtin_memcpy(&t.c[1], &c1, 16);
  t.s = (uint32_t)sc;
}

// The 8 activation fragments of k-tile kt for each 16-row block (packed
// activations); lanes whose row is >= M, or `ok` false, read zeros.
template <int MB>
__device__ inline void load_afrag(bf16x8 (&b)[MB][8], __amdgpu_buffer_rsrc_t ra, int kt, bool ok,
                                  int M, int lane) {
  const int col = lane & 15;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const bool v = ok && mb * 16 + col < M;
    const int base = v ? (kt * MB + mb) * 8 * ACT_FRAG_BYTES + lane * 16 : OOB;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(ra, base + q * ACT_FRAG_BYTES, 0, 0);
      __builtin_memcpy(&b[mb][q], &x, 16);
    }
  }
}

template <int MB>
__device__ inline void compute_wtile(const WTile &t, const bf16x8 (&b)[MB][8], f32x4 (&acc)[MB]) {
  float s[4];
  scales4(t.s, s);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const uint32_t cw[4] = {t.c[c].x, t.c[c].y, t.c[c].z, t.c[c].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 wf = dequant8(cw[j], s[2 * c + (j >> 1)]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, b[mb][4 * c + j], acc[mb], 0, 0, 0);
    }
  }
}

// Occupancy target (waves per SIMD) for the register allocator.
template <int MB, int R>
constexpr int waves_per_simd() {
  return MB == 1 ? 3 : 2;
}

__device__ inline uint16_t bf16_bits(float x) {
  const __hip_bfloat16 b = __float2bfloat16(x);  // round to nearest even
  uint16_t u;
  __builtin_memcpy(&u, &b, 2);
  return u;
}

__device__ inline float glue_pair(float g, float u, float c) {
#pragma clang fp contract(off)
  const float pg = g * c;
  const float pu = u * c;
  return pg + pu;
}

// Four consecutive bf16 outputs (column j, j % 4 == 0) of row m: into the next
// GEMM's packed activations and the optional row-major copies.
__device__ inline void store_next(const Epilogue &epi, int mblocks, int m, int j, int cols,
                                  const float (&o)[4]) {
  const uint32_t lo = (uint32_t)bf16_bits(o[0]) | ((uint32_t)bf16_bits(o[1]) << 16);
  const uint32_t hi = (uint32_t)bf16_bits(o[2]) | ((uint32_t)bf16_bits(o[3]) << 16);
  const uint2 v = make_uint2(lo, hi);
  *reinterpret_cast<uint2 *>(epi.act + act_offset(m, j, mblocks)) = v;
  if (epi.rm0) *reinterpret_cast<uint2 *>(epi.rm0 + (size_t)m * cols + j) = v;
  if (epi.rm1) *reinterpret_cast<uint2 *>(epi.rm1 + (size_t)m * cols + j) = v;
}

// Final values of the work-group's tiles are red[w][r][mb][l] summed over the
// first nw slots (wave order). Writes C (times ts) and the fused glue.
template <int MB, int R>
__device__ inline void epilogue(const f32x4 *red, int nw, int tid, int M, int N, int nrt, int rt0,
                                float ts, float *C, const Epilogue &epi) {
  if (epi.mode == EPI_PAIR) {
    const int half = N / 2;
    for (int it = tid; it < (R / 2) * MB * 64; it += WG_THREADS) {
      const int p = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      f32x4 vg = red[((0 * R + 2 * p) * MB + mb) * 64 + l];
      f32x4 vu = red[((0 * R + 2 * p + 1) * MB + mb) * 64 + l];
      for (int wv = 1; wv < nw; ++wv) {
        vg += red[((wv * R + 2 * p) * MB + mb) * 64 + l];
        vu += red[((wv * R + 2 * p + 1) * MB + mb) * 64 + l];
      }
      const int m = mb * 16 + (l & 15), rtg = rt0 + 2 * p;
      if (m >= M || rtg + 1 >= nrt) continue;
      const int j0 = (rtg / 2) * ROWS_PER_TILE + 4 * (l >> 4);
      if (j0 >= half) continue;
      vg *= ts;
      vu *= ts;
      if (epi.write_c) {
        *reinterpret_cast<f32x4 *>(C + (size_t)m * N + j0) = vg;
        *reinterpret_cast<f32x4 *>(C + (size_t)m * N + half + j0) = vu;
      }
      const float o[4] = {glue_pair(vg[0], vu[0], epi.c), glue_pair(vg[1], vu[1], epi.c),
                          glue_pair(vg[2], vu[2], epi.c), glue_pair(vg[3], vu[3], epi.c)};
      store_next(epi, MB, m, j0, half, o);
    }
    return;
  }
  for (int it = tid; it < R * MB * 64; it += WG_THREADS) {
    const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
    f32x4 v = red[((0 * R + r) * MB + mb) * 64 + l];
    for (int wv = 1; wv < nw; ++wv) v += red[((wv * R + r) * MB + mb) * 64 + l];
    // lane l of a tile holds D[n = 16 rt + 4 (l / 16) + i][m = 16 mb + l % 16]
    const int m = mb * 16 + (l & 15);
    const int rt = rt0 + r;
    const int n0 = rt * ROWS_PER_TILE + 4 * (l >> 4);
    if (m >= M || rt >= nrt || n0 >= N) continue;
    v *= ts;
    if (epi.write_c) {
      float *dst = C + (size_t)m * N + n0;
      if ((N & 3) == 0) {
        *reinterpret_cast<f32x4 *>(dst) = v;
      } else {
        for (int i = 0; i < 4; ++i)
          if (n0 + i < N) dst[i] = v[i];
      }
    }
    if (epi.mode == EPI_SCALE && n0 >= epi.col0 && n0 < epi.col1) {
      const float o[4] = {v[0] * epi.c, v[1] * epi.c, v[2] * epi.c, v[3] * epi.c};
      store_next(epi, MB, m, n0 - epi.col0, epi.col1 - epi.col0, o);
    }
  }
}

// ABUF = 2 double-buffers the activation fragments; with ABUF = 1 the next
// k-tile's fragments are loaded after the last use of the current ones (large
// M, where two copies do not fit in registers).
template <int MB, int R, int ABUF>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(waves_per_simd<MB, R>())))
void k_gemm(const uint8_t *__restrict__ act, int M, int act_bytes, const uint8_t *__restrict__ W,
            int N, int nrt, int nkt, int kts_per_split, int ksplit, float ts,
            float *__restrict__ C, float *__restrict__ part, unsigned *__restrict__ counters,
            Epilogue epi) {
  extern __shared__ __align__(16) f32x4 red[];  // [WG_WAVES][R][MB][64]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int rb = blockIdx.x, ks = blockIdx.y;
  const int rt0 = rb * R;
  const int kA = ks * kts_per_split;
  const int kB = min(nkt, kA + kts_per_split);
  const int len = kB - kA;
  const int kbeg = kA + (len * wave) / WG_WAVES;
  const int n = kA + (len * (wave + 1)) / WG_WAVES - kbeg;  // k-tiles of this wave
  const int stripe_bytes = nkt * TILE_BYTES;

  // One buffer resource per row tile (a row tile past the matrix has no
  // records, so its loads return zeros), one for the packed activations.
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    const uint8_t *base = W + (size_t)min(rt, nrt - 1) * (size_t)stripe_bytes;
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, rt < nrt ? stripe_bytes : 0,
                                              RAW_BUFFER_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, act_bytes, RAW_BUFFER_FLAGS);

  f32x4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  WTile w[R];
  bf16x8 a0[MB][8];
  load_afrag<MB>(a0, ra, kbeg, n > 0, M, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) load_wtile(w[r], rs[r], kbeg, n > 0, lane);
  if constexpr (ABUF == 2) {
    bf16x8 a1[MB][8];
    load_afrag<MB>(a1, ra, kbeg + 1, n > 1, M, lane);
    for (int i = 0; i < n; i += 2) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        compute_wtile<MB>(w[r], a0, acc[r]);
        load_wtile(w[r], rs[r], kbeg + i + 1, i + 1 < n, lane);
      }
      load_afrag<MB>(a0, ra, kbeg + i + 2, i + 2 < n, M, lane);
      if (i + 1 >= n) break;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        compute_wtile<MB>(w[r], a1, acc[r]);
        load_wtile(w[r], rs[r], kbeg + i + 2, i + 2 < n, lane);
      }
      load_afrag<MB>(a1, ra, kbeg + i + 3, i + 3 < n, M, lane);
    }
  } else {
    for (int i = 0; i < n; ++i) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        compute_wtile<MB>(w[r], a0, acc[r]);
        load_wtile(w[r], rs[r], kbeg + i + 1, i + 1 < n, lane);
      }
      load_afrag<MB>(a0, ra, kbeg + i + 1, i + 1 < n, M, lane);
    }
  }

  // Sum the 4 waves' tiles in wave order (LDS), then either finish here
  // (ksplit == 1) or exchange partial tiles with the other splits.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
  __syncthreads();

  const int npad = nrt * ROWS_PER_TILE;
  constexpr int ITEMS = R * MB * 64;
  int nw = WG_WAVES;
  if (ksplit > 1) {
    for (int it = tid; it < ITEMS; it += WG_THREADS) {
      const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      f32x4 v = red[((0 * R + r) * MB + mb) * 64 + l];
#pragma unroll
      for (int wv = 1; wv < WG_WAVES; ++wv) v += red[((wv * R + r) * MB + mb) * 64 + l];
      const int m = mb * 16 + (l & 15), rt = rt0 + r;
      if (m >= M || rt >= nrt) continue;
      float *dst = part + ((size_t)ks * M + m) * npad + rt * ROWS_PER_TILE + 4 * (l >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_store(dst + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // The partial stores have reached memory once this wave's counters drain.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ unsigned s_ticket;
    if (tid == 0)
      s_ticket = __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    if (s_ticket != (unsigned)(ksplit - 1)) return;
    // Last to arrive: sum the splits in order 0..ksplit-1 into slot 0.
    for (int it = tid; it < ITEMS; it += WG_THREADS) {
      const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      const int m = mb * 16 + (l & 15), rt = rt0 + r;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m < M && rt < nrt) {
        const float *src = part + (size_t)m * npad + rt * ROWS_PER_TILE + 4 * (l >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        for (int s2 = 1; s2 < ksplit; ++s2) {
          const float *s2p = src + (size_t)s2 * M * npad;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v[i] += __hip_atomic_load(s2p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
      }
      red[((0 * R + r) * MB + mb) * 64 + l] = v;
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    nw = 1;
  }
  epilogue<MB, R>(red, nw, tid, M, N, nrt, rt0, ts, C, epi);
}

typedef void (*GemmKernel)(const uint8_t *, int, int, const uint8_t *, int, int, int, int, int,
                           float, float *, float *, unsigned *, Epilogue);

GemmKernel pick_kernel(int mb, int r) {
  switch (mb * 16 + r) {
    case 1 * 16 + 1: return k_gemm<1, 1, 2>;
    case 1 * 16 + 2: return k_gemm<1, 2, 2>;
    case 1 * 16 + 4: return k_gemm<1, 4, 2>;
    case 1 * 16 + 8: return k_gemm<1, 8, 2>;
    case 2 * 16 + 1: return k_gemm<2, 1, 2>;
    case 2 * 16 + 2: return k_gemm<2, 2, 2>;
    case 2 * 16 + 4: return k_gemm<2, 4, 2>;
    case 2 * 16 + 8: return k_gemm<2, 8, 1>;
    case 3 * 16 + 1: return k_gemm<3, 1, 1>;
    case 3 * 16 + 2: return k_gemm<3, 2, 1>;
    case 3 * 16 + 4: return k_gemm<3, 4, 1>;
    case 4 * 16 + 1: return k_gemm<4, 1, 1>;
    case 4 * 16 + 2: return k_gemm<4, 2, 1>;
    case 4 * 16 + 4: return k_gemm<4, 4, 1>;
    default: return nullptr;
  }
}

// Row-major A -> packed activations: one thread per 16-byte chunk.
__global__ void k_pack_act(const uint16_t *__restrict__ A, int M, int K, int mblocks, int nkt,
                           uint4 *__restrict__ out) {
  const int64_t total = (int64_t)nkt * mblocks * 8 * 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  const int64_t frag = idx >> 6;  // (kt * MB + mb) * 8 + q
  const int q = (int)(frag & 7);
  const int64_t kt_mb = frag >> 3;
  const int mb = (int)(kt_mb % mblocks);
  const int64_t kt = kt_mb / mblocks;
  const int row = mb * 16 + (lane & 15);
  const int64_t k0 = kt * K_PER_TILE + 64 * (lane >> 4) + 8 * q;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < M && k0 < K) v = *reinterpret_cast<const uint4 *>(A + (size_t)row * K + k0);
  out[idx] = v;
}

}  // namespace

namespace nvfp4v {

// Tile table for gfx950, from a sweep of R (row tiles per work-group, sharing
// one activation fragment) and ksplit (work-groups along K) over the layer
// shapes [15360|5120|34816 x 5120], [5120 x 17408] and [151936 x 5120] at
// M = 1, 16, 32, 64 (median of 9 timed launches over 1 GiB of rotated weight
// copies each):
//  * splitting K across work-groups only pays for K-heavy, narrow matrices
//    (down: 3 splits); everywhere else one work-group covers all of K;
//  * R = 2 is best up to about 4096 row tiles at M <= 32; very wide matrices
//    (the 151936-row head) want R = 4 at M <= 16 and R = 8 at M <= 32;
//  * at M > 32, R = 4 except for the narrowest matrices (R = 2).
// NVFP4V_PLAN="r=<R>,ks=<ksplit>" overrides both (used by tuning sweeps).
int make_plan(const nvfp4v_ctx *ctx, const Layout &L, int64_t m, Plan *p) {
  p->mblocks = (int)((m + 15) / 16);
  p->waves = WG_WAVES;
  const int64_t nrt = L.nrt;
  const int nkt = (int)L.nkt;
  if (p->mblocks == 1)
    p->rb = nrt >= 4096 && m > 1 ? 4 : 2;
  else if (p->mblocks == 2)
    p->rb = nrt >= 4096 ? 8 : 2;
  else
    p->rb = nrt >= 640 ? 4 : 2;
  int want_ks = (nkt >= 48 && nrt <= 640) ? 3 : 1;
  if (const char *ov = std::getenv("NVFP4V_PLAN")) {
    int r = 0, k2 = 0;
    if (std::sscanf(ov, "r=%d,ks=%d", &r, &k2) == 2 && (r == 1 || r == 2 || r == 4 || r == 8)) {
      p->rb = r;
      want_ks = k2 > 0 ? k2 : 1;
    }
  }
  (void)ctx;
  int force_ks = want_ks;
  if (!pick_kernel(p->mblocks, p->rb)) p->rb = 4;
  p->grid_x = (int)((L.nrt + p->rb - 1) / p->rb);
  {
    const int ks = std::min(force_ks, nkt);
    const int per = (nkt + ks - 1) / ks;
    p->ktiles_per_split = per;
    p->ksplit = p->grid_y = (nkt + per - 1) / per;
  }
  p->lds_bytes = (size_t)WG_WAVES * p->rb * p->mblocks * 64 * sizeof(f32x4);
  return NVFP4V_OK;
}

int launch_pack_act(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                    hipStream_t stream) {
  const int mb = (int)((m + 15) / 16), nkt = (int)((k + 255) / 256);
  const int64_t total = (int64_t)nkt * mb * 8 * 64;
  hipLaunchKernelGGL(k_pack_act, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a,
                     (int)m, (int)k, mb, nkt, (uint4 *)act);
  return hip_status(ctx, hipGetLastError());
}

int launch_gemm(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                int64_t n, float ts, float *c, hipStream_t stream, const Epilogue &epi) {
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  Plan p;
  int rc = make_plan(ctx, L, m, &p);
  if (rc) return rc;
  if (epi.mode == EPI_PAIR && (p.rb & 1)) {  // (gate, up) row-tile pairs need an even R
    p.rb = 2;
    p.grid_x = (int)((L.nrt + p.rb - 1) / p.rb);
    p.lds_bytes = (size_t)WG_WAVES * p.rb * p.mblocks * 64 * sizeof(f32x4);
  }
  if (p.ksplit > 1) {
    const size_t need = (size_t)p.ksplit * (size_t)m * (size_t)(L.nrt * ROWS_PER_TILE);
    if (need > ctx->partial_floats || (size_t)p.grid_x > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  }
  GemmKernel kern = pick_kernel(p.mblocks, p.rb);
  if (!kern) return NVFP4V_E_INVALID_ARG;
  if (fault_injected()) return NVFP4V_E_FAULT;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.grid_x, (unsigned)p.grid_y), dim3(WG_THREADS),
                     p.lds_bytes, stream, act, (int)m, (int)act_packed_bytes(m, k),
                     (const uint8_t *)packed, (int)n, (int)L.nrt, (int)L.nkt, p.ktiles_per_split,
                     p.ksplit, ts, c, ctx->partials, ctx->counters, epi);
  return hip_status(ctx, hipGetLastError());
}

}  // namespace nvfp4v

extern "C" size_t nvfp4v_act_packed_bytes(int64_t m, int64_t k) {
  if (m < 1 || m > NVFP4V_MAX_M || k < 16 || k % 16 != 0 || k > (int64_t(1) << 22)) return 0;
  return act_packed_bytes(m, k);
}

extern "C" int nvfp4v_pack_activations(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k,
                                       void *act, hipStream_t stream) {
  if (!ctx || !a || !act) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  if (k < 16 || k % 16 != 0 || k > (int64_t(1) << 22)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(act)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  return launch_pack_act(ctx, a, m, k, (uint8_t *)act, stream);
}

extern "C" int nvfp4v_verify_gemm_pa(nvfp4v_ctx *ctx, const void *act, int64_t m, int64_t k,
                                     const void *packed, int64_t n, float ts, float *c,
                                     hipStream_t stream) {
  if (!ctx || !act || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(act) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  return launch_gemm(ctx, (const uint8_t *)act, m, k, packed, n, ts, c, stream);
}

extern "C" int nvfp4v_verify_gemm(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k,
                                  const void *packed, int64_t n, float ts, float *c,
                                  hipStream_t stream) {
  if (!ctx || !a || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  if (act_packed_bytes(m, k) > ctx->act_bytes) return NVFP4V_E_WORKSPACE;
  Plan p;
  int rc = make_plan(ctx, L, m, &p);
  if (rc) return rc;
  if (p.ksplit > 1) {
    const size_t need = (size_t)p.ksplit * (size_t)m * (size_t)(L.nrt * ROWS_PER_TILE);
    if (need > ctx->partial_floats || (size_t)p.grid_x > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  }
  if (fault_injected()) return NVFP4V_E_FAULT;
  rc = launch_pack_act(ctx, a, m, k, ctx->act, stream);
  if (rc) return rc;
  return launch_gemm(ctx, ctx->act, m, k, packed, n, ts, c, stream);
}

extern "C" int nvfp4v_describe_plan(nvfp4v_ctx *ctx, int64_t n, int64_t k, int64_t m, char *buf,
                                    size_t len) {
  if (!ctx || !buf || len == 0) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  Plan p;
  int rc = make_plan(ctx, L, m, &p);
  if (rc) return rc;
  snprintf(buf, len, "mfma16x16x32 mblocks=%d r=%d waves=%d grid=%dx%d ksplit=%d kt/split=%d lds=%zu",
           p.mblocks, p.rb, p.waves, p.grid_x, p.grid_y, p.ksplit, p.ktiles_per_split, p.lds_bytes);
  return NVFP4V_OK;
}
