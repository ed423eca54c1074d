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
//  * Dequantisation is exact, in fp16: v_cvt_scalef32_pk_f16_fp4 turns two
//    E2M1 codes into fp16 (with a unit scale; on gfx950 the instruction applies
//    only the exponent of its scale operand) and one v_pk_mul_f16 applies the
//    E4M3 block scale, decoded to fp16 (an E2M1 value times an E4M3 scale has
//    at most 6 significant bits and lies in [2^-10, 2688]): one VALU operation
//    per weight.
//  * v_mfma_f32_16x16x32_f16 with the weights as the 16-row A operand and a
//    16-row block of activations as the B operand, fp32 accumulation. The
//    activations come from the fp16 copy of the packed activations (internal.h:
//    the bf16 values times 2^8, exact, or a NaN marker where fp16 cannot hold
//    the value), so every product is exact and the sums are the bf16 products'
//    sums times 2^8, scaled back at the end of the unit. A unit whose sums hold
//    a NaN is computed again from the bf16 copy with the bf16 form of the
//    dequantisation (v_cvt_scalef32_pk_f32_fp4, two fp32 multiplies, the high
//    halves packed as bf16) and v_mfma_f32_16x16x32_bf16: C is bitwise what the
//    bf16 path alone gives (on gfx950 the two MFMAs sum the same exact
//    products identically).
//  * The 4 waves' tiles are summed through LDS in wave order. With ksplit > 1
//    the K pieces of a row block exchange partial tiles. By default (the
//    create-time dispatch probe found that work-groups with linear ids
//    congruent mod 8 run on one XCD, and the grid's x is padded to a multiple
//    of 8) they meet in that XCD's L2: plain stores, a ticket atomic executed
//    in the L2, loads that read through the L1. In the register variant the
//    last piece to take a ticket sums the partials; in the LDS variant the
//    row block's last piece is a designated reducer that keeps its own
//    partial in LDS and waits for its siblings. Otherwise (or with
//    NVFP4V_SPLITK_EXCHANGE=memory) they meet in memory: system-coherent
//    stores, ticket and loads, and the last arriver sums. Every path sums in
//    split order 0..ksplit-1, so C is bitwise reproducible and the two
//    exchanges agree bitwise (TandemLLM manual, 1.7 "The paper": the 4-bit
//    kernels keep a fixed reduction order). No float atomics.
#include <algorithm>
#include <cctype>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gemm_device.h"

using namespace nvfp4v;

namespace {

using namespace nvfp4v::dev;

template <int MB, int R, int D, bool A2 = false>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(waves_per_simd<MB, R, D, A2>())))
void k_gemm(GemmArgs g) {
  extern __shared__ __align__(16) f32x4 red[];
  if ((int)blockIdx.x >= g.nrb) return;  // grid padding
  if (g.xcd_local && blockIdx.y == 0 && threadIdx.x == 0) count_row_block(g.status, DEV_ROWS_BEGUN);
  const int ks = blockIdx.y, kA = ks * g.kts_per_split, kB = min(g.nkt, kA + g.kts_per_split);
  // Every kernel carries both paths (its registers are the larger path's):
  // the fp16 copy first, the bf16 copy for a unit that met a marker.
  if (g.act16 && gemm_unit<MB, R, D, A2, true>(g, blockIdx.x, kA, kB, ks, g.ksplit, red)) return;
  count_f16_redone(g);
  gemm_unit<MB, R, D, A2, false>(g, blockIdx.x, kA, kB, ks, g.ksplit, red);
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
  if (g.act16 && gemm_unit_lds<MB, R, true>(g, blockIdx.x, blockIdx.y, lds)) return;
  count_f16_redone(g);
  gemm_unit_lds<MB, R, false>(g, blockIdx.x, blockIdx.y, lds);
}

// The wide-M variant: 1 wave per SIMD with 4 row tiles per wave, 2 with 2.
template <int MB, int R>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(R >= 4 ? 1 : 2)))
void k_gemm_wide(GemmArgs g) {
  extern __shared__ __align__(16) uint8_t lds[];
  if ((int)blockIdx.x >= g.nrb) return;  // grid padding
  if (g.xcd_local && blockIdx.y == 0 && threadIdx.x == 0) count_row_block(g.status, DEV_ROWS_BEGUN);
  if (g.act16 && gemm_unit_wide<MB, R, true>(g, blockIdx.x, blockIdx.y, lds)) return;
  count_f16_redone(g);
  gemm_unit_wide<MB, R, false>(g, blockIdx.x, blockIdx.y, lds);
}

typedef void (*GemmKernel)(GemmArgs);

GemmKernel pick_wide_kernel(int mb, int r) {
  switch (mb * 16 + r) {
    case 3 * 16 + 2: return k_gemm_wide<3, 2>;
    case 4 * 16 + 2: return k_gemm_wide<4, 2>;
    case 5 * 16 + 2: return k_gemm_wide<5, 2>;
    case 6 * 16 + 2: return k_gemm_wide<6, 2>;
    case 7 * 16 + 2: return k_gemm_wide<7, 2>;
    case 8 * 16 + 2: return k_gemm_wide<8, 2>;
    case 4 * 16 + 4: return k_gemm_wide<4, 4>;
    case 8 * 16 + 4: return k_gemm_wide<8, 4>;
    default: return nullptr;
  }
}

// LDS of the wide variant: one k-tile of activations, or the work-group's
// tile sums (which reuse it) if larger, plus the ticket slot.
size_t wide_variant_bytes(int mb, int r) {
  return std::max((size_t)mb * 8 * ACT_FRAG_BYTES, (size_t)WG_WAVES * r * mb * 64 * sizeof(f32x4)) + 16;
}

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
// The one-deep ring with two-deep activation fragments (gemm_unit's A2) for
// four row tiles at two row blocks (in place of the one-deep ring) and at one
// (in place of the two-deep ring: it fits three waves per SIMD, 0.4-0.6 %
// faster over the pass at 9..16 rows); NVFP4V_A2=0 keeps the plain rings.
static bool use_a2() {
  const char *ov = std::getenv("NVFP4V_A2");
  return !ov || std::atoi(ov) != 0;
}

GemmKernel pick_kernel(int mb, int r, int d) {
  if (mb == 2 && r == 4 && d == 1 && use_a2()) return k_gemm<2, 4, 1, true>;
  if (mb == 1 && r == 4 && d == 2 && use_a2()) return k_gemm<1, 4, 1, true>;
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

// Row-major A -> packed activations: one thread per 16-byte chunk, into the
// bf16 copy and, when act16 > 0, the fp16 copy act16 / 16 chunks further on.
// `sync` (optional): the persistent pass's barrier words, zeroed here because
// this kernel starts every pass (its grid always has more threads than words).
__global__ void k_pack_act(const uint16_t *__restrict__ A, int M, int K, int mblocks, int nkt,
                           uint4 *__restrict__ out, int64_t act16, unsigned *sync) {
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
  if (act16) {
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      h[i] = (uint32_t)f16_act_bits((uint16_t)(in[i] & 0xFFFFu)) |
             ((uint32_t)f16_act_bits((uint16_t)(in[i] >> 16)) << 16);
    out[idx + act16 / 16] = make_uint4(h[0], h[1], h[2], h[3]);
  }
}

}  // namespace

namespace nvfp4v {

// ---------------------------------------------------------------------------
// Tile table. The built-in table is the library's tables/gfx950.txt, compiled
// in (the build embeds the file); a context may load another file, whose rules
// are tried first. The rows were measured on MI355X (see the file's header).
// ---------------------------------------------------------------------------
static const char kBuiltinTable[] =
#include "tile_table_gfx950.inc"
    ;

// A field of a rule: a non-negative integer, or "*" (returns `open`).
static bool parse_bound(const char *tok, int open, int *out) {
  if (std::strcmp(tok, "*") == 0) {
    *out = open;
    return true;
  }
  char *end = nullptr;
  const long v = std::strtol(tok, &end, 10);
  if (!end || *end != 0 || v < 0 || v > (1L << 30)) return false;
  *out = (int)v;
  return true;
}

// Every M of the rule's range has a compiled kernel for its kernel and R.
static bool rule_has_kernels(const TileRule &t) {
  for (int mb = (t.m_lo + 15) / 16; mb <= (t.m_hi + 15) / 16; ++mb) {
    const bool ok = t.lds == 2 ? pick_wide_kernel(mb, t.r) != nullptr
                  : t.lds == 1 ? pick_lds_kernel(mb, t.r) != nullptr
                               : ring_depth(mb, t.r, 4) != 0;
    if (!ok) return false;
  }
  return true;
}

int parse_tile_table(const char *text, TileRule *rules, int *n_rules) {
  int n = 0;
  bool arch_ok = false;
  const char *p = text;
  while (*p) {
    const char *eol = std::strchr(p, '\n');
    const size_t len = eol ? (size_t)(eol - p) : std::strlen(p);
    std::string line(p, len);
    p = eol ? eol + 1 : p + len;
    const size_t hash = line.find('#');
    if (hash != std::string::npos) line.resize(hash);
    std::vector<std::string> tok;
    size_t i = 0;
    while (i < line.size()) {
      while (i < line.size() && std::isspace((unsigned char)line[i])) ++i;
      size_t j = i;
      while (j < line.size() && !std::isspace((unsigned char)line[j])) ++j;
      if (j > i) tok.emplace_back(line.substr(i, j - i));
      i = j;
    }
    if (tok.empty()) continue;
    if (tok[0] == "arch") {
      if (tok.size() != 2 || tok[1] != "gfx950") return NVFP4V_E_TABLE;
      arch_ok = true;
      continue;
    }
    if (tok[0] != "rule" || tok.size() != 10 || n >= MAX_TILE_RULES) return NVFP4V_E_TABLE;
    TileRule t;
    if (!parse_bound(tok[1].c_str(), 1, &t.nrt_lo) || !parse_bound(tok[2].c_str(), 1 << 30, &t.nrt_hi) ||
        !parse_bound(tok[3].c_str(), 1, &t.nkt_lo) || !parse_bound(tok[4].c_str(), 1 << 30, &t.nkt_hi) ||
        !parse_bound(tok[5].c_str(), 1, &t.m_lo) || !parse_bound(tok[6].c_str(), NVFP4V_MAX_M, &t.m_hi))
      return NVFP4V_E_TABLE;
    if (tok[7] == "wide") t.lds = 2;
    else if (tok[7] == "lds") t.lds = 1;
    else if (tok[7] == "reg") t.lds = 0;
    else return NVFP4V_E_TABLE;
    if (!parse_bound(tok[8].c_str(), 0, &t.r) || !parse_bound(tok[9].c_str(), 0, &t.ksplit)) return NVFP4V_E_TABLE;
    if (t.nrt_lo < 1 || t.nrt_lo > t.nrt_hi || t.nkt_lo < 1 || t.nkt_lo > t.nkt_hi || t.m_lo < 1 ||
        t.m_lo > t.m_hi || t.m_hi > (t.lds == 2 ? NVFP4V_MAX_M : CHUNK_M) || t.ksplit < 1 || t.ksplit > 64 ||
        !rule_has_kernels(t))
      return NVFP4V_E_TABLE;
    rules[n++] = t;
  }
  if (!arch_ok) return NVFP4V_E_TABLE;
  *n_rules = n;
  return NVFP4V_OK;
}

static const TileRule *find_rule(const TileRule *rules, int n, int64_t nrt, int64_t nkt, int64_t m) {
  for (int i = 0; i < n; ++i) {
    const TileRule &t = rules[i];
    if (nrt >= t.nrt_lo && nrt <= t.nrt_hi && nkt >= t.nkt_lo && nkt <= t.nkt_hi && m >= t.m_lo && m <= t.m_hi)
      return &t;
  }
  return nullptr;
}

static const TileRule *builtin_rules(int *n) {
  static TileRule rules[MAX_TILE_RULES];
  static int count = -1;
  if (count < 0) {
    int c = 0;
    count = parse_tile_table(kBuiltinTable, rules, &c) == NVFP4V_OK ? c : 0;
  }
  *n = count;
  return rules;
}

// NVFP4V_PLAN="r=<R>,ks=<ksplit>" (or "n:..." for the LDS variant) overrides
// the table (used by tuning sweeps).
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
  int want_ks = 1;
  int want_d = 2;
  p->lds = 0;
  p->rb = 2;
  const TileRule *rule = ctx && ctx->n_rules > 0 ? find_rule(ctx->rules, ctx->n_rules, nrt, nkt, m) : nullptr;
  if (!rule) {
    int nb = 0;
    const TileRule *b = builtin_rules(&nb);
    rule = find_rule(b, nb, nrt, nkt, m);
  }
  if (rule) {
    p->lds = rule->lds;
    p->rb = rule->r;
    want_ks = rule->ksplit;
  }
  if (const char *ov = std::getenv("NVFP4V_PLAN")) {
    int r = 0, k2 = 0;
    if (std::sscanf(ov, "w:r=%d,ks=%d", &r, &k2) == 2 && pick_wide_kernel(p->mblocks, r)) {
      p->lds = 2;
      p->rb = r;
      want_ks = k2 > 0 ? k2 : 1;
    } else if (std::sscanf(ov, "n:r=%d,ks=%d", &r, &k2) == 2 && pick_lds_kernel(p->mblocks, r)) {
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
  if (p->lds == 2 && !pick_wide_kernel(p->mblocks, p->rb)) p->lds = 0, p->rb = 2;
  if (p->lds == 1 && !pick_lds_kernel(p->mblocks, p->rb)) p->lds = 0, p->rb = 2;
  if (!p->lds && !ring_depth(p->mblocks, p->rb, 4)) p->rb = 4;
  p->depth = p->lds ? 0 : ring_depth(p->mblocks, p->rb, want_d);
  const int64_t rows_per_group = p->lds ? (int64_t)WG_WAVES * p->rb : p->rb;
  p->grid_x = (int)((L.nrt + rows_per_group - 1) / rows_per_group);
  {
    const int ks = std::min(want_ks, nkt);
    const int per = (nkt + ks - 1) / ks;
    p->ktiles_per_split = per;
    p->ksplit = p->grid_y = (nkt + per - 1) / per;
  }
  p->lds_bytes = p->lds == 2 ? wide_variant_bytes(p->mblocks, p->rb)
                : p->lds    ? lds_variant_bytes(p->mblocks, p->rb)
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

bool use_f16() {
  const char *ov = std::getenv("NVFP4V_F16");
  return !ov || std::atoi(ov) != 0;
}

int launch_pack_act(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                    size_t act16, hipStream_t stream, unsigned *sync) {
  const int mb = (int)((m + 15) / 16), nkt = (int)((k + 255) / 256);
  const int64_t total = (int64_t)nkt * mb * 8 * 64;
  int64_t blocks = (total + 255) / 256;
  if (sync) blocks = std::max<int64_t>(blocks, (PASS_SYNC_WORDS + 255) / 256);
  hipLaunchKernelGGL(k_pack_act, dim3((unsigned)blocks), dim3(256), 0, stream, a, (int)m, (int)k,
                     mb, nkt, (uint4 *)act, (int64_t)act16, sync);
  return hip_status(ctx, hipGetLastError());
}

int launch_gemm(nvfp4v_ctx *ctx, const uint8_t *act, size_t act16, int64_t m, int64_t k,
                const void *packed, int64_t n, float ts, float *c, hipStream_t stream,
                const Epilogue &epi) {
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
  GemmKernel kern = p.lds == 2 ? pick_wide_kernel(p.mblocks, p.rb)
                  : p.lds      ? pick_lds_kernel(p.mblocks, p.rb)
                               : pick_kernel(p.mblocks, p.rb, p.depth);
  if (!kern) return NVFP4V_E_INVALID_ARG;
  if (m > CHUNK_M && p.lds != 2) return NVFP4V_E_INVALID_ARG;  // only the wide unit takes > 64 rows
  if (fault_injected()) return NVFP4V_E_FAULT;
  GemmArgs g;
  g.act = act;
  g.M = (int)m;
  g.act_bytes = (int)act_copy_bytes(m, k);
  g.act16 = (int)act16;
  g.act_blk1 = m > CHUNK_M ? (int)act_block_bytes(CHUNK_M, k) : 0;
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

// Whether the tile table gives an M-row call (M > 64) one launch of the wide
// unit over both packed blocks of rows.
static bool wide_rows(const nvfp4v_ctx *ctx, int64_t m, int64_t k, int64_t n) {
  if (m <= CHUNK_M) return false;
  Layout L;
  Plan p;
  return make_layout(n, k, &L) && make_plan(ctx, L, m, &p) == NVFP4V_OK && p.lds == 2;
}

int launch_gemm_rows(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                     int64_t n, float ts, float *c, hipStream_t stream) {
  const size_t act16 = use_f16() ? act_copy_bytes(m, k) : 0;
  if (wide_rows(ctx, m, k, n)) return launch_gemm(ctx, act, act16, m, k, packed, n, ts, c, stream);
  int rc = NVFP4V_OK;
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    rc = launch_gemm(ctx, act, act16, mc, k, packed, n, ts, c + r0 * n, stream);
    act += act_block_bytes(mc, k);
  }
  return rc;
}

int launch_pack_rows(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                     hipStream_t stream) {
  const size_t act16 = act_copy_bytes(m, k);
  int rc = NVFP4V_OK;
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    rc = launch_pack_act(ctx, a + r0 * k, mc, k, act, act16, stream);
    act += act_block_bytes(mc, k);
  }
  return rc;
}

// Workspace checks of the plan of every block of rows of an M-row call.
static int check_rows_workspace(const nvfp4v_ctx *ctx, const Layout &L, int64_t m) {
  const bool wide = wide_rows(ctx, m, L.k, L.n);
  for (int64_t r0 = 0; r0 < m; r0 += CHUNK_M) {
    const int64_t mc = wide ? m : std::min<int64_t>(CHUNK_M, m - r0);
    if (wide && r0 > 0) break;
    Plan p;
    const int rc = make_plan(ctx, L, mc, &p);
    if (rc) return rc;
    if (p.ksplit > 1) {
      const size_t need = (size_t)p.ksplit * (size_t)mc * (size_t)(L.nrt * ROWS_PER_TILE);
      if (need > ctx->partial_floats || (size_t)p.nrb > ctx->n_counters) return NVFP4V_E_WORKSPACE;
    }
  }
  return NVFP4V_OK;
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
  return launch_pack_rows(ctx, a, m, k, (uint8_t *)act, stream);
}

extern "C" int nvfp4v_verify_gemm_pa(nvfp4v_ctx *ctx, const void *act, int64_t m, int64_t k,
                                     const void *packed, int64_t n, float ts, float *c,
                                     hipStream_t stream) {
  if (!ctx || !act || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(act) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  const int rc = check_rows_workspace(ctx, L, m);
  if (rc) return rc;
  if (fault_injected()) return NVFP4V_E_FAULT;
  return launch_gemm_rows(ctx, (const uint8_t *)act, m, k, packed, n, ts, c, stream);
}

extern "C" int nvfp4v_verify_gemm(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k,
                                  const void *packed, int64_t n, float ts, float *c,
                                  hipStream_t stream) {
  if (!ctx || !a || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  if (2 * act_block_bytes(std::min<int64_t>(m, CHUNK_M), k) > ctx->act_bytes) return NVFP4V_E_WORKSPACE;
  int rc = check_rows_workspace(ctx, L, m);
  if (rc) return rc;
  if (fault_injected()) return NVFP4V_E_FAULT;
  // All rows packed at once when they fit the context's buffer, so that more
  // than 64 rows can take the wide unit's single launch; else one block of
  // rows at a time (stream order keeps a block's GEMM ahead of the next
  // block's packing).
  if (act_packed_bytes(m, k) <= ctx->act_bytes) {
    rc = launch_pack_rows(ctx, a, m, k, ctx->act, stream);
    return rc ? rc : launch_gemm_rows(ctx, ctx->act, m, k, packed, n, ts, c, stream);
  }
  const bool f16 = use_f16();
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    const size_t act16 = act_block_bytes(mc, k);
    rc = launch_pack_act(ctx, a + r0 * k, mc, k, ctx->act, act16, stream);
    if (!rc) rc = launch_gemm(ctx, ctx->act, f16 ? act16 : 0, mc, k, packed, n, ts, c + r0 * n, stream);
  }
  return rc;
}

extern "C" int nvfp4v_load_tile_table(nvfp4v_ctx *ctx, const char *path) {
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  if (!path) {
    ctx->n_rules = 0;
    return NVFP4V_OK;
  }
  FILE *f = std::fopen(path, "rb");
  if (!f) return NVFP4V_E_TABLE;
  std::string text;
  char buf[4096];
  size_t got;
  while ((got = std::fread(buf, 1, sizeof(buf), f)) > 0 && text.size() < (1u << 20)) text.append(buf, got);
  std::fclose(f);
  if (text.size() >= (1u << 20)) return NVFP4V_E_TABLE;
  TileRule rules[MAX_TILE_RULES];
  int n = 0;
  const int rc = parse_tile_table(text.c_str(), rules, &n);
  if (rc) return rc;
  std::memcpy(ctx->rules, rules, sizeof(TileRule) * (size_t)n);
  ctx->n_rules = n;
  return NVFP4V_OK;
}

extern "C" int nvfp4v_describe_plan(nvfp4v_ctx *ctx, int64_t n, int64_t k, int64_t m, char *buf,
                                    size_t len) {
  if (!ctx || !buf || len == 0) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  // M > 64 runs one launch of the wide unit if the table says so, else one
  // launch per block of 64 rows: then the first block's plan and the number
  // of launches.
  const bool wide = wide_rows(ctx, m, k, n);
  const int64_t blocks = wide ? 1 : (m + CHUNK_M - 1) / CHUNK_M;
  Plan p;
  int rc = make_plan(ctx, L, wide ? m : std::min<int64_t>(m, CHUNK_M), &p);
  if (rc) return rc;
  char blk[48] = "";
  if (blocks > 1) snprintf(blk, sizeof(blk), " launches=%lld (64-row blocks)", (long long)blocks);
  snprintf(buf, len, "mfma16x16x32 %s mblocks=%d r=%d depth=%d waves=%d grid=%dx%d ksplit=%d kt/split=%d lds=%zu exchange=%s%s",
           p.lds == 2 ? "wide-m/waves-split-n" : p.lds ? "act-in-lds/waves-split-n" : "waves-split-k", p.mblocks,
           p.rb, p.depth, p.waves,
           p.grid_x, p.grid_y, p.ksplit, p.ktiles_per_split, p.lds_bytes,
           p.ksplit == 1 ? "none" : p.xcd_local ? "xcd-l2" : "memory", blk);
  return NVFP4V_OK;
}
