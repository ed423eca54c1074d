// The verify GEMM: C[M][N] = ts * A[M][K] * W[N][K]^T with W in the packed
// NVFP4 layout (internal.h), M = 1..64, on gfx950.
//
// Work decomposition. A work-group of 4 waves owns a row block of 4 row tiles
// (64 weight rows) and one split of the k-tiles; each wave streams one row
// tile across the split. The work-group stages the activations of the k-chunk
// it is working on in LDS (all M rows, bf16), so each activation byte is read
// from L2 once per work-group and reused by all four waves.
//
// Per k-tile a lane loads its 16 code bytes and 2 scale bytes, dequantises
// 8 codes at a time to bf16 (exact: an E2M1 value times an E4M3 scale has at
// most 6 significant bits and lies in [2^-10, 2688]) and issues one
// v_mfma_f32_16x16x32_bf16 per 8 codes and per 16-row block of M: the weights
// are the MFMA's A operand (16 rows), the activations its B operand (16
// columns), fp32 accumulation.
//
// Split-K. With ksplit > 1, every work-group writes its fp32 partial tile to
// the context workspace and takes an arrival ticket; the last work-group of
// the row block sums the partials in split order 0..ksplit-1 (a fixed order,
// independent of arrival order; no float atomics) and writes C. This keeps the
// K-reduction order fixed, as the pages require of the 4-bit kernels
// (TandemLLM manual, "What TandemLLM is", 1.7 "The paper").
#include <algorithm>
#include <cstdio>

#include "internal.h"

using namespace nvfp4v;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WG_THREADS = 256;
constexpr int WG_WAVES = 4;
constexpr int LDS_BUDGET = 40 * 1024;  // per work-group: 4 work-groups fit one CU's 160 KiB

// E4M3 byte -> fp32, exact (NaN for 0x7F / 0xFF).
__device__ inline float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0)
    v = (float)m * 0.001953125f;  // m * 2^-9
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  return (b & 0x80u) ? -v : v;
}

template <int SEL>
__device__ inline uint32_t dq_pair(uint32_t codes, float s) {
  // Two E2M1 codes (byte SEL: low nibble = even k) -> two fp32, times s, then the
  // high halves packed as bf16x2 (exact, the products fit bf16).
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

__device__ inline bf16x8 lds_b(const uint16_t *p) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int MB>
__global__ __launch_bounds__(WG_THREADS) void k_gemm_mfma(
    const uint16_t *__restrict__ A, int M, int K, const uint8_t *__restrict__ W, int N, int nrt,
    int nkt, int kts_per_split, int kts_per_chunk, int ksplit, float ts, float *__restrict__ C,
    float *__restrict__ part, unsigned *__restrict__ counters) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane >> 4, col = lane & 15;
  const int rb = blockIdx.x, ks = blockIdx.y;
  const int kt0 = ks * kts_per_split;
  const int kt1 = min(nkt, kt0 + kts_per_split);
  const int rt = rb * WG_WAVES + wave;
  const bool active = rt < nrt;
  const uint8_t *stripe = W + (size_t)(active ? rt : 0) * (size_t)nkt * TILE_BYTES;

  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = kt0; c0 < kt1; c0 += kts_per_chunk) {
    const int c1 = min(kt1, c0 + kts_per_chunk);
    const int kspan = (c1 - c0) * K_PER_TILE;
    const int pitch = kspan + 8;  // bf16 elements; 16-byte pad staggers LDS banks
    // Stage A[0..M)[c0*128 .. c0*128 + kspan) (zeros beyond K).
    const int cpr = kspan / 8;  // 16-byte chunks per row
    __syncthreads();            // previous chunk fully consumed
    for (int c = tid; c < M * cpr; c += WG_THREADS) {
      const int m = c / cpr, kc = c - m * cpr;
      const int kg = c0 * K_PER_TILE + kc * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (kg < K) v = *reinterpret_cast<const uint4 *>(A + (size_t)m * K + kg);
      *reinterpret_cast<uint4 *>(lds + m * pitch + kc * 8) = v;
    }
    __syncthreads();
    if (active) {
      for (int kt = c0; kt < c1; ++kt) {
        const int g = kt >> 3, t = kt & 7;
        const int q = min(TILES_PER_GROUP, nkt - g * TILES_PER_GROUP);
        const uint8_t *grp = stripe + (size_t)g * TILES_PER_GROUP * TILE_BYTES;
        const uint4 cw = *reinterpret_cast<const uint4 *>(grp + t * CODE_TILE_BYTES + lane * 16);
        const uint32_t sc =
            *reinterpret_cast<const uint16_t *>(grp + q * CODE_TILE_BYTES + lane * 2 * q + 2 * t);
        const float s0 = e4m3_to_f32(sc & 0xFFu), s1 = e4m3_to_f32(sc >> 8);
        const bf16x8 w0 = dequant8(cw.x, s0), w1 = dequant8(cw.y, s0);
        const bf16x8 w2 = dequant8(cw.z, s1), w3 = dequant8(cw.w, s1);
        const int kl = (kt - c0) * K_PER_TILE + 32 * h;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int m = mb * 16 + col;
          bf16x8 b0, b1, b2, b3;
          if (m < M) {
            const uint16_t *ap = lds + m * pitch + kl;
            b0 = lds_b(ap);
            b1 = lds_b(ap + 8);
            b2 = lds_b(ap + 16);
            b3 = lds_b(ap + 24);
          } else {
            b0 = b1 = b2 = b3 = bf16x8{};
          }
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, b0, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, b1, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2, b2, acc[mb], 0, 0, 0);
          acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w3, b3, acc[mb], 0, 0, 0);
        }
      }
    }
  }

  // Lane (h, col) holds D[n = 16 rt + 4h + i][m = 16 mb + col], i = 0..3.
  const int npad = nrt * ROWS_PER_TILE;
  const int n0 = rt * ROWS_PER_TILE + 4 * h;
  if (ksplit == 1) {
    if (active) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = mb * 16 + col;
        if (m >= M) continue;
        float *dst = C + (size_t)m * N + n0;
        if ((N & 3) == 0) {
          if (n0 < N) *reinterpret_cast<f32x4 *>(dst) = acc[mb] * ts;
        } else {
          for (int i = 0; i < 4; ++i)
            if (n0 + i < N) dst[i] = acc[mb][i] * ts;
        }
      }
    }
    return;
  }

  if (active) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = mb * 16 + col;
      if (m < M) *reinterpret_cast<f32x4 *>(part + ((size_t)ks * M + m) * npad + n0) = acc[mb];
    }
  }
  __threadfence();
  __syncthreads();
  __shared__ unsigned s_ticket;
  if (tid == 0) s_ticket = atomicAdd(&counters[rb], 1u);
  __syncthreads();
  if (s_ticket != (unsigned)(ksplit - 1)) return;
  __threadfence();
  const int rows = WG_WAVES * ROWS_PER_TILE;
  for (int e = tid; e < M * rows; e += WG_THREADS) {
    const int m = e / rows, n = rb * rows + (e - m * rows);
    if (n >= N) continue;
    float sum = 0.f;
    for (int s = 0; s < ksplit; ++s) sum += part[((size_t)s * M + m) * npad + n];
    C[(size_t)m * N + n] = sum * ts;
  }
  if (tid == 0) counters[rb] = 0u;  // ready for the next launch
}

}  // namespace

namespace nvfp4v {

int make_plan(const nvfp4v_ctx *ctx, const Layout &L, int64_t m, Plan *p) {
  p->variant = 0;
  p->mblocks = (int)((m + 15) / 16);
  p->waves = WG_WAVES;
  p->row_tiles_per_wg = WG_WAVES;
  p->grid_x = (int)((L.nrt + WG_WAVES - 1) / WG_WAVES);
  const int nkt = (int)L.nkt;
  // k-tiles per LDS chunk for this M
  const int per_row = LDS_BUDGET / (2 * (int)m);
  int chunk = (per_row - 8) / K_PER_TILE;
  chunk = std::max(1, std::min(chunk, nkt));
  // split K so that about 4 work-groups per CU are in flight
  const int target = 4 * std::max(1, ctx->num_cus);
  int ks = std::max(1, (target + p->grid_x - 1) / p->grid_x);
  ks = std::min(ks, nkt);
  int per = (nkt + ks - 1) / ks;
  ks = (nkt + per - 1) / per;
  p->ksplit = ks;
  p->ktiles_per_split = per;
  p->grid_y = ks;
  // an LDS chunk never spans more than the split
  p->ktiles_per_chunk = std::min(chunk, per);
  p->lds_bytes = (size_t)m * (size_t)(p->ktiles_per_chunk * K_PER_TILE + 8) * 2;
  return NVFP4V_OK;
}

}  // namespace nvfp4v

extern "C" int nvfp4v_verify_gemm(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k,
                                  const void *packed, int64_t n, float ts, float *c,
                                  hipStream_t stream) {
  if (!ctx || !a || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  Plan p;
  int rc = make_plan(ctx, L, m, &p);
  if (rc) return rc;
  if (p.ksplit > 1) {
    const size_t need = (size_t)p.ksplit * (size_t)m * (size_t)(L.nrt * ROWS_PER_TILE);
    if (need > ctx->partial_floats || (size_t)p.grid_x > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  }
  if (fault_injected()) return NVFP4V_E_FAULT;
  const dim3 grid((unsigned)p.grid_x, (unsigned)p.grid_y);
  const dim3 block(WG_THREADS);
#define LAUNCH(MBV)                                                                               \
  hipLaunchKernelGGL(k_gemm_mfma<MBV>, grid, block, p.lds_bytes, stream, a, (int)m, (int)k,      \
                     (const uint8_t *)packed, (int)n, (int)L.nrt, (int)L.nkt, p.ktiles_per_split, \
                     p.ktiles_per_chunk, p.ksplit, ts, c, ctx->partials, ctx->counters)
  switch (p.mblocks) {
    case 1: LAUNCH(1); break;
    case 2: LAUNCH(2); break;
    case 3: LAUNCH(3); break;
    default: LAUNCH(4); break;
  }
#undef LAUNCH
  return hip_status(ctx, hipGetLastError());
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
  snprintf(buf, len, "mfma16x16x32 mblocks=%d waves=%d rows/wg=%d grid=%dx%d ksplit=%d kt/split=%d kt/chunk=%d lds=%zu",
           p.mblocks, p.waves, p.row_tiles_per_wg * ROWS_PER_TILE, p.grid_x, p.grid_y, p.ksplit,
           p.ktiles_per_split, p.ktiles_per_chunk, p.lds_bytes);
  return NVFP4V_OK;
}
