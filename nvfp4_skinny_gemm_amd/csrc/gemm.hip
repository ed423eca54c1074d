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
#include <cstring>
#include <vector>

#include "gemm_device.h"

using namespace nvfp4v;

namespace {

using namespace nvfp4v::dev;

template <int MB, int R, int D>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(waves_per_simd<MB, R, D>())))
void k_gemm(GemmArgs g) {
  extern __shared__ __align__(16) f32x4 red[];
  if ((int)blockIdx.x >= g.nrb) return;  // grid padding
  if (g.xcd_local && blockIdx.y == 0 && threadIdx.x == 0) count_row_block(g.status, DEV_ROWS_BEGUN);
  const int ks = blockIdx.y, kA = ks * g.kts_per_split;
  gemm_unit<MB, R, D>(g, blockIdx.x, kA, min(g.nkt, kA + g.kts_per_split), ks, g.ksplit, red);
}

template <int MB, int R>
constexpr int lds_waves_per_simd() {
  return MB == 1 ? (R == 1 ? 4 : 3) : 2;
}

template <int MB, int R>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(lds_waves_per_simd<MB, R>())))
void k_gemm_lds(GemmArgs g) {
  extern __shared__ __align__(16) uint8_t lds[];
  if ((int)blockIdx.x >= g.nrb) return;  // grid padding
  if (g.xcd_local && blockIdx.y == 0 && threadIdx.x == 0) count_row_block(g.status, DEV_ROWS_BEGUN);
  gemm_unit_lds<MB, R>(g, blockIdx.x, blockIdx.y, lds);
}

typedef void (*GemmKernel)(GemmArgs);

GemmKernel pick_lds_kernel(int mb, int r) {
  switch (mb * 16 + r) {
    case 1 * 16 + 1: return k_gemm_lds<1, 1>;
    case 1 * 16 + 2: return k_gemm_lds<1, 2>;
    case 2 * 16 + 1: return k_gemm_lds<2, 1>;
    case 2 * 16 + 2: return k_gemm_lds<2, 2>;
    case 3 * 16 + 1: return k_gemm_lds<3, 1>;
    case 4 * 16 + 1: return k_gemm_lds<4, 1>;
    default: return nullptr;
  }
}

size_t lds_variant_bytes(int mb, int r) {
  return (size_t)2 * mb * 8 * ACT_FRAG_BYTES + (size_t)WG_WAVES * r * mb * 64 * sizeof(f32x4) + 16;
}

// Ring depth per (row blocks, R): 2 by default, 1 where two copies of the
// fragments do not fit. Depths 3-4 are reachable only through NVFP4V_PLAN
// (measured slower in the pass at 1-16 rows, kept for the override's tests).
GemmKernel pick_kernel(int mb, int r, int d) {
  switch ((mb * 16 + r) * 8 + d) {
    case (1 * 16 + 1) * 8 + 2: return k_gemm<1, 1, 2>;
    case (1 * 16 + 2) * 8 + 2: return k_gemm<1, 2, 2>;
    case (1 * 16 + 2) * 8 + 3: return k_gemm<1, 2, 3>;
    case (1 * 16 + 2) * 8 + 4: return k_gemm<1, 2, 4>;
    case (1 * 16 + 4) * 8 + 2: return k_gemm<1, 4, 2>;
    case (1 * 16 + 4) * 8 + 3: return k_gemm<1, 4, 3>;
    case (1 * 16 + 8) * 8 + 1: return k_gemm<1, 8, 1>;
    case (2 * 16 + 1) * 8 + 2: return k_gemm<2, 1, 2>;
    case (2 * 16 + 2) * 8 + 2: return k_gemm<2, 2, 2>;
    case (2 * 16 + 4) * 8 + 1: return k_gemm<2, 4, 1>;
    case (2 * 16 + 8) * 8 + 1: return k_gemm<2, 8, 1>;
    case (3 * 16 + 1) * 8 + 1: return k_gemm<3, 1, 1>;
    case (3 * 16 + 2) * 8 + 1: return k_gemm<3, 2, 1>;
    case (3 * 16 + 4) * 8 + 1: return k_gemm<3, 4, 1>;
    case (4 * 16 + 1) * 8 + 1: return k_gemm<4, 1, 1>;
    case (4 * 16 + 2) * 8 + 1: return k_gemm<4, 2, 1>;
    case (4 * 16 + 4) * 8 + 1: return k_gemm<4, 4, 1>;
    default: return nullptr;
  }
}

// The deepest ring compiled for (row blocks, R), capped at `want`.
int ring_depth(int mb, int r, int want) {
  for (int d = want; d >= 1; --d)
    if (pick_kernel(mb, r, d)) return d;
  return 0;
}

// Dispatch probe: every work-group records the XCD it runs on.
__global__ void k_xcd_probe(unsigned *out) {
  if (threadIdx.x == 0)
    out[blockIdx.x + blockIdx.y * gridDim.x] = (unsigned)__builtin_amdgcn_s_getreg(XCC_ID_HWREG) & 0xFu;
}

// Row-major A -> packed activations: one thread per 16-byte chunk.
// `sync` (optional): the persistent pass's barrier words, zeroed here because
// this kernel starts every pass (its grid always has more threads than words).
__global__ void k_pack_act(const uint16_t *__restrict__ A, int M, int K, int mblocks, int nkt,
                           uint4 *__restrict__ out, unsigned *sync) {
  const int64_t total = (int64_t)nkt * mblocks * 8 * 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (sync && idx < PASS_SYNC_WORDS) sync[idx] = 0u;
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

// Tile table for gfx950. R = row tiles per wave item sharing one activation
// fragment, ksplit = work-groups along K, "LDS" = the variant whose waves
// split N and share activations staged in LDS. From sweeps of R in {1,2,4,8}
// x ksplit in {1,2,3,4,6,8} x both variants, one projection at a time, inside
// the graph-replayed 64-layer pass (the other projections at their chosen
// plans), at M = 1, 8, 9, 16, 17, 24, 32, and of single launches over 1 GiB
// of rotated weight copies for the LM head and M > 32:
//  * up to 8 rows: R = 2 everywhere, K split 3 for the K-heavy narrow down
//    projection [5120 x 17408];
//  * 9..16 rows (twice the activation bytes per k-tile): R = 4 for q|k|v (960
//    row tiles), LDS with K split 3 from 1024 row tiles (gate|up: 2176 in the
//    pass, 1088 for one of the pair alone, 15 % faster than R = 4 there), LDS
//    with K split 6 for down, R = 2 for o;
//  * 17..32 rows: R = 4 with K split 3 for down, R = 4 for q|k|v and gate|up,
//    R = 2 for o;
//  * the 151936-row LM head: LDS with R = 2 per wave up to 32 rows;
//  * beyond 32 rows: R = 4 with K split 3 for down, and for the narrow
//    square matrices beyond 48 rows; R = 2 for those up to 48 rows; R = 4
//    for the wide ones.
// Split-K exchanges meet in one XCD's L2 (unit_tail), which is what makes the
// K splits at 9..16 rows pay.
// NVFP4V_PLAN="r=<R>,ks=<ksplit>" overrides both (used by tuning sweeps).
static void finish_grid(const nvfp4v_ctx *ctx, Plan *p) {
  p->nrb = p->grid_x;
  p->xcd_local = p->ksplit > 1 && ctx && ctx->xcd_local;
  if (p->xcd_local) p->grid_x = (p->grid_x + 7) & ~7;
}

int make_plan(const nvfp4v_ctx *ctx, const Layout &L, int64_t m, Plan *p) {
  p->mblocks = (int)((m + 15) / 16);
  p->waves = WG_WAVES;
  const int64_t nrt = L.nrt;
  const int nkt = (int)L.nkt;
  const bool narrow = nrt <= 640, deep = nkt >= 48;  // o and down vs q|k|v and gate|up
  int want_ks = 1;
  p->lds = 0;
  int want_d = 2;
  if (p->mblocks == 1) {
    p->rb = nrt >= 4096 && m > 1 ? 4 : 2;
    if (deep && narrow) {
      want_ks = 3;
      if (m > 8) p->lds = 1, p->rb = 1, want_ks = 6;
    } else if (m > 8 && !narrow && nrt < 4096) {
      if (nrt >= 1024) p->lds = 1, p->rb = 1, want_ks = 3;
      else p->rb = 4;
    }
  } else if (p->mblocks == 2) {
    p->rb = nrt >= 4096 ? 8 : narrow && !deep ? 2 : 4;
    if (deep && narrow) want_ks = 3;
  } else {
    p->rb = nrt >= 640 || deep || p->mblocks == 4 ? 4 : 2;
    if (narrow && (deep || p->mblocks == 4)) want_ks = 3;
  }
  // The LM head up to 32 rows: activations staged in LDS, R = 2 per wave.
  if (p->mblocks <= 2 && nrt >= 4096) p->lds = 1, p->rb = 2, want_ks = 1;
  if (const char *ov = std::getenv("NVFP4V_PLAN")) {
    int r = 0, k2 = 0;
    if (std::sscanf(ov, "n:r=%d,ks=%d", &r, &k2) == 2 && pick_lds_kernel(p->mblocks, r)) {
      p->lds = 1;
      p->rb = r;
      want_ks = k2 > 0 ? k2 : 1;
    } else if (std::sscanf(ov, "r=%d,ks=%d", &r, &k2) == 2 && (r == 1 || r == 2 || r == 4 || r == 8)) {
      int d2 = 0;
      p->lds = 0;
      p->rb = r;
      want_ks = k2 > 0 ? k2 : 1;
      if (std::sscanf(ov, "r=%*d,ks=%*d,d=%d", &d2) == 1 && d2 >= 1) want_d = d2;
    }
  }
  int force_ks = want_ks;
  if (!p->lds && !ring_depth(p->mblocks, p->rb, 4)) p->rb = 4;
  p->depth = p->lds ? 0 : ring_depth(p->mblocks, p->rb, want_d);
  const int64_t rows_per_group = p->lds ? (int64_t)WG_WAVES * p->rb : p->rb;
  p->grid_x = (int)((L.nrt + rows_per_group - 1) / rows_per_group);
  {
    const int ks = std::min(force_ks, nkt);
    const int per = (nkt + ks - 1) / ks;
    p->ktiles_per_split = per;
    p->ksplit = p->grid_y = (nkt + per - 1) / per;
  }
  p->lds_bytes = p->lds ? lds_variant_bytes(p->mblocks, p->rb)
                       : (size_t)WG_WAVES * p->rb * p->mblocks * 64 * sizeof(f32x4) + 16;
  finish_grid(ctx, p);
  return NVFP4V_OK;
}

// The split-K exchange through one XCD's L2 needs the work-groups whose
// linear ids are congruent mod 8 to run on one XCD: gfx950 in its one-partition
// mode deals the work-groups of a dispatch out to its XCDs round-robin by id
// (the XCD that takes id 0 can differ between queues, which is harmless).
// This launches grids of the shapes the GEMM uses and checks exactly that
// property in each; if a launch breaks it (another partition mode or device),
// the context keeps the exchange through memory. At run time the GEMM counts
// the row blocks begun and completed, and nvfp4v_device_status reports a
// difference. NVFP4V_SPLITK_EXCHANGE=memory forces the exchange through memory.
int probe_dispatch(nvfp4v_ctx *ctx) {
  ctx->xcd_local = 0;
  const char *env = std::getenv("NVFP4V_SPLITK_EXCHANGE");
  if (env && std::strcmp(env, "memory") == 0) return NVFP4V_OK;
  static const int shapes[][2] = {{4096, 1}, {8, 512}, {240, 2}, {1088, 3}, {160, 3}, {16, 9}, {80, 6}};
  unsigned *buf = reinterpret_cast<unsigned *>(ctx->partials);  // free before the first GEMM
  std::vector<unsigned> h(4096);
  bool ok = true;
  for (const auto &sh : shapes) {
    const int n = sh[0] * sh[1];
    hipError_t e = hipMemset(buf, 0xFF, (size_t)n * sizeof(unsigned));
    if (e == hipSuccess) {
      hipLaunchKernelGGL(k_xcd_probe, dim3((unsigned)sh[0], (unsigned)sh[1]), dim3(64), 0, 0, buf);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpy(h.data(), buf, (size_t)n * sizeof(unsigned), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(ctx, e);
    for (int i = 0; i < n && ok; ++i) ok = h[i] <= 15u && h[i] == h[i & 7];
  }
  ctx->xcd_local = ok ? 1 : 0;
  return NVFP4V_OK;
}

int launch_pack_act(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                    hipStream_t stream, unsigned *sync) {
  const int mb = (int)((m + 15) / 16), nkt = (int)((k + 255) / 256);
  const int64_t total = (int64_t)nkt * mb * 8 * 64;
  int64_t blocks = (total + 255) / 256;
  if (sync) blocks = std::max<int64_t>(blocks, (PASS_SYNC_WORDS + 255) / 256);
  hipLaunchKernelGGL(k_pack_act, dim3((unsigned)blocks), dim3(256), 0, stream, a, (int)m, (int)k,
                     mb, nkt, (uint4 *)act, sync);
  return hip_status(ctx, hipGetLastError());
}

int launch_gemm(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                int64_t n, float ts, float *c, hipStream_t stream, const Epilogue &epi) {
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  Plan p;
  int rc = make_plan(ctx, L, m, &p);
  if (rc) return rc;
  if (!p.lds && epi.mode == EPI_PAIR && (p.rb & 1)) {  // (gate, up) row-tile pairs need an even R
    p.rb = 2;
    p.depth = ring_depth(p.mblocks, 2, p.depth);
    p.grid_x = (int)((L.nrt + p.rb - 1) / p.rb);
    p.lds_bytes = (size_t)WG_WAVES * p.rb * p.mblocks * 64 * sizeof(f32x4) + 16;
    finish_grid(ctx, &p);
  }
  if (p.ksplit > 1) {
    const size_t need = (size_t)p.ksplit * (size_t)m * (size_t)(L.nrt * ROWS_PER_TILE);
    if (need > ctx->partial_floats || (size_t)p.nrb > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  }
  GemmKernel kern = p.lds ? pick_lds_kernel(p.mblocks, p.rb) : pick_kernel(p.mblocks, p.rb, p.depth);
  if (!kern) return NVFP4V_E_INVALID_ARG;
  if (fault_injected()) return NVFP4V_E_FAULT;
  GemmArgs g;
  g.act = act;
  g.M = (int)m;
  g.act_bytes = (int)act_packed_bytes(m, k);
  g.W = (const uint8_t *)packed;
  g.N = (int)n;
  g.nrt = (int)L.nrt;
  g.nkt = (int)L.nkt;
  g.kts_per_split = p.ktiles_per_split;
  g.ksplit = p.ksplit;
  g.ts = ts;
  g.C = c;
  g.part = ctx->partials;
  g.counters = ctx->counters;
  g.epi = epi;
  g.nrb = p.nrb;
  g.xcd_local = p.xcd_local;
  g.status = ctx->dev_status;
  hipLaunchKernelGGL(kern, dim3((unsigned)p.grid_x, (unsigned)p.grid_y), dim3(WG_THREADS),
                     p.lds_bytes, stream, g);
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
    if (need > ctx->partial_floats || (size_t)p.nrb > ctx->n_counters) return NVFP4V_E_WORKSPACE;
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
  snprintf(buf, len, "mfma16x16x32 %s mblocks=%d r=%d depth=%d waves=%d grid=%dx%d ksplit=%d kt/split=%d lds=%zu exchange=%s",
           p.lds ? "act-in-lds/waves-split-n" : "waves-split-k", p.mblocks, p.rb, p.depth, p.waves,
           p.grid_x, p.grid_y, p.ksplit, p.ktiles_per_split, p.lds_bytes,
           p.ksplit == 1 ? "none" : p.xcd_local ? "xcd-l2" : "memory");
  return NVFP4V_OK;
}
