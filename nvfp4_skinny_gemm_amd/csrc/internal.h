// Internal declarations of the nvfp4v library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstring>

#include "../../include/nvfp4v.h"

// ---------------------------------------------------------------------------
// Packed (device) layout.
//
// The weight matrix is cut into row tiles of 16 rows; each row tile is one
// contiguous stripe over all of K, cut into k-tiles of 256 elements:
//
//   tile(rt, kt)  = (rt * nkt + kt) * TILE_BYTES            (2304 bytes)
//   code half c   : bytes [1024 c, 1024 c + 1024), c = 0, 1; lane L = r + 16h
//                   (r = row in tile, h = 0..3) owns 16 bytes at 16 L: the 32
//                   codes of row r for k in [256 kt + 64 h + 32 c, +32), in
//                   canonical order (byte b: low nibble k = 2b, high 2b + 1)
//   scales        : bytes [2048 + 4 L, 2048 + 4 L + 4): byte e is the E4M3
//                   scale of row r, 16-block 16 kt + 4 h + e
//
// A wave reads a tile with three fully coalesced loads (2 x 1 KiB of codes,
// 256 bytes of scales). Dword j of code half c holds the 8 codes the lane
// feeds to MFMA (c, j) of the tile, and its scale is byte 2c + j/2. Each byte
// of the canonical format appears once; padding (rows >= N, k >= K) is zero
// codes with zero scales, which contributes exact zeros.
// ---------------------------------------------------------------------------
namespace nvfp4v {

constexpr int ROWS_PER_TILE = 16;
constexpr int K_PER_TILE = 256;
constexpr int CODE_HALF_BYTES = 1024;
constexpr int SCALE_OFFSET = 2048;
constexpr int TILE_BYTES = 2304;

struct Layout {
  int64_t n, k;
  int64_t nrt;  // row tiles
  int64_t nkt;  // k tiles
  size_t bytes() const { return (size_t)nrt * (size_t)nkt * TILE_BYTES; }
};

// Activations in MFMA fragment order ("packed activations"): for k-tile kt,
// 16-row block mb and fragment q = 0..7, a 1 KiB chunk at
//   ((kt * MB + mb) * 8 + q) * 1024
// whose lane L = col + 16 h holds 8 values A[16 mb + col][256 kt + 64 h + 8 q + e],
// e = 0..7 (MB = ceil(M / 16)). A wave reads one fragment with one fully
// coalesced 16-byte load per lane. Rows >= M are read only where a work-group
// stages whole blocks (the verify GEMM's staged variants with two or more
// row blocks, the FP8 head), and their sums are never stored; every other
// loader gets zeros for them from an out-of-range offset.
//
// The packed form holds two copies of A in this order: the bf16 values, and
// `act16` bytes further on (the size of one copy) the same values as fp16
// times 2^ACT_F16_SHIFT. A bf16 value converts to fp16 exactly when it is 0 or
// its magnitude lies in [2^(-17-S), 2^(16-S)) (S = the shift; fp16 keeps all 8
// significant bits there, as a normal or subnormal number); any other value
// (too small or large, inf, NaN) is stored in the fp16 copy as the NaN
// ACT_F16_MARK. The GEMM takes the fp16 copy: its products of exact fp16
// weights and exact fp16 activations are the bf16 path's products times 2^S,
// so the fp32 sums are too (measured on MI355X: v_mfma_f32_16x16x32_f16 and
// _bf16 on the same values agree bitwise), and the sums are scaled back
// exactly. A marker turns the sums it enters into NaN (NaN times zero is NaN
// in both MFMAs), and a unit whose sums hold a NaN is computed again from the
// bf16 copy, so every result equals the bf16 path's.
constexpr int ACT_FRAG_BYTES = 1024;
constexpr int ACT_F16_SHIFT = 8;
constexpr uint16_t ACT_F16_MARK = 0x7FFF;

// Words of the persistent pass's barrier block (context memory).
constexpr int PASS_SYNC_WORDS = 1280;

// One GEMM launch takes at most CHUNK_M rows. Activations of more rows (a
// verify pass over several sequences' trees) are packed as consecutive blocks
// of CHUNK_M rows, the last one shorter, each block in the layout above for
// its own row count; a GEMM over them runs once per block.
constexpr int CHUNK_M = 64;

// Bytes of one copy of one block of rows.
inline size_t act_block_bytes(int64_t m, int64_t k) {
  const int64_t mb = (m + 15) / 16, nkt = (k + 255) / 256;
  return (size_t)nkt * (size_t)mb * 8 * ACT_FRAG_BYTES;
}

// Bytes of one copy (all blocks of rows): the distance from the bf16 copy to
// the fp16 copy of packed activations written for all m rows at once.
inline size_t act_copy_bytes(int64_t m, int64_t k) {
  size_t total = 0;
  for (int64_t r0 = 0; r0 < m; r0 += CHUNK_M) total += act_block_bytes(m - r0 < CHUNK_M ? m - r0 : CHUNK_M, k);
  return total;
}

// Bytes of the packed form (both copies).
inline size_t act_packed_bytes(int64_t m, int64_t k) { return 2 * act_copy_bytes(m, k); }

// Byte offset of element (row, col) of A inside the packed activations.
__host__ __device__ inline size_t act_offset(int64_t row, int64_t k, int mblocks) {
  const int64_t kt = k >> 8, rem = k & 255;
  const int64_t h = rem >> 6, q = (rem >> 3) & 7, e = rem & 7;
  const int64_t mb = row >> 4, col = row & 15;
  return (size_t)(((kt * mblocks + mb) * 8 + q) * ACT_FRAG_BYTES + (col + 16 * h) * 16 + 2 * e);
}

inline bool make_layout(int64_t n, int64_t k, Layout *L) {
  if (n < 1 || k < 16 || k % 16 != 0) return false;
  if (n > (int64_t(1) << 31) || k > (int64_t(1) << 22)) return false;  // keeps 32-bit buffer offsets in range
  L->n = n;
  L->k = k;
  L->nrt = (n + ROWS_PER_TILE - 1) / ROWS_PER_TILE;
  L->nkt = (k + K_PER_TILE - 1) / K_PER_TILE;
  return true;
}

// ---------------------------------------------------------------------------
// Format encoders shared by the host and device quantisers (product side).
// ---------------------------------------------------------------------------

// Round a finite, non-negative double to the nearest E4M3 magnitude (ties to
// even), saturating at 448, by integer rounding of the fp64 significand.
__host__ __device__ inline uint32_t e4m3_encode_mag(double x) {
  if (!(x < 448.0)) return 0x7E;
  uint64_t bits;
  memcpy(&bits, &x, 8);
  const int bexp = (int)((bits >> 52) & 0x7FF);
  if (bexp == 0) return 0;  // zero or fp64 subnormal: far below 2^-10
  const int e = bexp - 1023;
  uint64_t sig = (bits & ((uint64_t(1) << 52) - 1)) | (uint64_t(1) << 52);  // value = sig * 2^(e-52)
  // Target grid step: 2^(e-3) for e >= -6 (3 stored mantissa bits), 2^-9 below.
  const int step = e >= -6 ? e - 3 : -9;
  const int shift = step - (e - 52);  // drop `shift` low bits of sig
  if (shift > 60) return 0;           // below half of 2^-9: rounds to 0
  const uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((uint64_t(1) << shift) - 1);
  const uint64_t half = uint64_t(1) << (shift - 1);
  uint64_t r = q + ((rem > half || (rem == half && (q & 1))) ? 1 : 0);
  // r is the value in units of 2^step.
  if (e < -6) return (uint32_t)r;  // 0..8 (8 = 2^-6, the same bit pattern as e=1,m=0)
  int ef = e + 7;
  if (r == 16) {
    r = 8;
    ef += 1;
  }
  const uint32_t out = ((uint32_t)ef << 3) | (uint32_t)(r - 8);
  return out > 0x7E ? 0x7E : out;
}

__host__ __device__ inline double e4m3_decode_f64(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  double v;
  if (e == 15 && m == 7) return __builtin_nan("");
  if (e == 0)
    v = (double)m * (1.0 / 512.0);
  else {
    // 2^(e-7) * (8 + m) / 8
    uint64_t bits = ((uint64_t)(e - 7 + 1023) << 52) | ((uint64_t)m << 49);
    memcpy(&v, &bits, 8);
  }
  return (b & 0x80) ? -v : v;
}

// E2M1 round-to-nearest (ties to the even mantissa), saturating at 6, sign kept.
__host__ __device__ inline uint32_t e2m1_encode(double q) {
  const uint32_t sgn = __builtin_signbit(q) ? 8u : 0u;
  const double a = q < 0 ? -q : q;
  uint32_t c;
  if (a <= 0.25) c = 0;
  else if (a < 0.75) c = 1;
  else if (a <= 1.25) c = 2;
  else if (a < 1.75) c = 3;
  else if (a <= 2.5) c = 4;
  else if (a < 3.5) c = 5;
  else if (a <= 5.0) c = 6;
  else c = 7;
  return c | sgn;
}

// Quantise one 16-element block: writes 8 code bytes and returns the scale byte.
__host__ __device__ inline uint32_t quantize_block(const float *w, uint8_t *codes8) {
  double amax = 0.0;
  for (int t = 0; t < 16; ++t) {
    const double a = w[t] < 0 ? -(double)w[t] : (double)w[t];
    amax = a > amax ? a : amax;
  }
  const uint32_t sb = e4m3_encode_mag(amax / 6.0);
  const double s = e4m3_decode_f64(sb);
  for (int b = 0; b < 8; ++b) {
    uint32_t lo = 0, hi = 0;
    if (s != 0.0) {
      lo = e2m1_encode((double)w[2 * b] / s);
      hi = e2m1_encode((double)w[2 * b + 1] / s);
    }
    codes8[b] = (uint8_t)(lo | (hi << 4));
  }
  return sb;
}

// ---------------------------------------------------------------------------
// Context.
// ---------------------------------------------------------------------------
struct Plan {
  int mblocks;           // ceil(M / 16): 16-column MFMA blocks of activations
  int lds;               // 0: waves split the k-range, each loads its own activation
                         //    fragments; 1: waves split N, activations staged in LDS
  int rb;                // row tiles per wave item (variant 0: per work-group; 1: per wave)
  int waves;             // waves per work-group
  int depth;             // variant 0: k-tiles in flight per wave (its register ring)
  int ksplit;            // work-groups along K (fixed-order reduction when > 1)
  int ktiles_per_split;  // k-tiles per work-group
  int grid_x, grid_y;    // row blocks (padded to a multiple of 8 with xcd_local), k splits
  size_t lds_bytes;      // cross-wave reduction buffer
  int nrb;               // row blocks
  int xcd_local;         // split-K exchange through one XCD's L2 (else through memory)
};

// One row of a tile table: GEMMs with row tiles in [nrt_lo, nrt_hi], k-tiles
// in [nkt_lo, nkt_hi] and M in [m_lo, m_hi] take this plan.
struct TileRule {
  int nrt_lo, nrt_hi, nkt_lo, nkt_hi, m_lo, m_hi;
  int lds;     // 1: the LDS-staged variant
  int r;       // row tiles per work-group (reg) or per wave (lds)
  int ksplit;  // work-groups along K
};
constexpr int MAX_TILE_RULES = 64;

}  // namespace nvfp4v

struct nvfp4v_ctx {
  int device = 0;
  int num_cus = 0;
  int last_hip = 0;
  float *partials = nullptr;  // split-K partial sums
  size_t partial_floats = 0;
  unsigned *counters = nullptr;  // per row-block arrival counters (kept at 0 between calls)
  size_t n_counters = 0;
  uint8_t *act = nullptr;  // packed activations for nvfp4v_verify_gemm
  size_t act_bytes = 0;
  unsigned *pass_sync = nullptr;  // persistent pass: barrier arrivals, finished groups, error flag
  int pass_mode = NVFP4V_PASS_CHAIN;
  int last_pass_grid = 0;         // work-groups of the last persistent pass launch
  uint64_t *pass_timeline = nullptr;  // optional (NVFP4V_PASS_TRACE=1): per phase and work-group,
                                      // real-time clock at phase start and at work done
  size_t pass_timeline_words = 0;
  int last_pass_phases = 0;
  int xcd_local = 0;  // the dispatch probe allows the split-K exchange through one XCD's L2
  unsigned *dev_status = nullptr;  // DEV_STATUS_BYTES: row-block counts of that exchange
  // Tile table loaded from a file (nvfp4v_load_tile_table), tried before the
  // built-in one; none when n_rules == 0 (an all-zero context uses the
  // built-in table).
  int n_rules = 0;
  nvfp4v::TileRule rules[nvfp4v::MAX_TILE_RULES];
};

// Context status lines: 8 lines of DEV_LINE_WORDS words, line x holding the
// row blocks begun and completed on XCD x by split-K GEMMs that exchange
// through one XCD's L2 (the two totals differ only if a row block's pieces
// ran on two XCDs), and the GEMM work units on XCD x computed again from the
// bf16 copy of their activations after meeting a marker in the fp16 copy.
constexpr int DEV_LINE_WORDS = 32, DEV_ROWS_BEGUN = 0, DEV_ROWS_DONE = 1, DEV_F16_REDONE = 2;
constexpr size_t DEV_STATUS_BYTES = 8 * DEV_LINE_WORDS * sizeof(unsigned);

// Timeline capacity: 2 stamps for each of up to 1024 work-groups and 512 phases.
constexpr size_t PASS_TIMELINE_WGS = 1024, PASS_TIMELINE_PHASES = 512;

namespace nvfp4v {
int fault_injected();  // NVFP4V_FAULT=launch
int hip_status(nvfp4v_ctx *ctx, hipError_t e);
bool aligned16(const void *p);
int make_plan(const nvfp4v_ctx *ctx, const Layout &L, int64_t m, Plan *p);
// Parse a tile table (text); NVFP4V_E_TABLE if it is malformed, names another
// arch or a kernel the library does not have.
int parse_tile_table(const char *text, TileRule *rules, int *n_rules);
// Sets ctx->xcd_local from a dispatch probe (synchronous; at create).
int probe_dispatch(nvfp4v_ctx *ctx);
// Enqueue A (row-major bf16, at most CHUNK_M rows) -> packed activations (no
// argument checks): the bf16 copy at `act` and, when act16 > 0, the fp16 copy
// act16 bytes further on.
int launch_pack_act(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                    size_t act16, hipStream_t stream, unsigned *sync = nullptr);
// Fused epilogue of a GEMM in the chained pass: besides (optionally) writing
// the fp32 C, turn C into the next GEMM's bf16 input, in packed-activation
// order, and optionally into up to two row-major bf16 copies.
//   EPI_NONE:  C only.
//   EPI_SCALE: for columns [col0, col1): out[m][j - col0] = bf16(C[m][j] * c).
//   EPI_PAIR:  row tiles come in (gate, up) pairs (tile 2t = gate rows
//              16t..16t+15, tile 2t+1 = the matching up rows);
//              out[m][j] = bf16(gate * c + up * c) (no fused multiply-add), and
//              C is written in natural order [gate | up].
enum EpiMode { EPI_NONE = 0, EPI_SCALE = 1, EPI_PAIR = 2 };
struct Epilogue {
  int mode = EPI_NONE;
  int col0 = 0, col1 = 0;
  float c = 1.f;
  uint8_t *act = nullptr;  // packed activations of the next GEMM (its K = out columns)
  int act16 = 0;           // > 0: also write their fp16 copy, act16 bytes after `act`
  uint16_t *rm0 = nullptr, *rm1 = nullptr;  // optional row-major bf16 copies [M][out cols]
  int write_c = 1;
};
// Enqueue the GEMM on packed activations (no argument checks; m <= CHUNK_M,
// or the wide unit's rows). act16 > 0: the fp16 copy lies act16 bytes after
// `act` and the GEMM computes from it; 0: from the bf16 copy.
int launch_gemm(nvfp4v_ctx *ctx, const uint8_t *act, size_t act16, int64_t m, int64_t k,
                const void *packed, int64_t n, float ts, float *c, hipStream_t stream,
                const Epilogue &epi = Epilogue());
// The same for any m over activations packed by launch_pack_rows: one launch
// per block of CHUNK_M rows, or one of the wide unit (plain epilogue).
int launch_gemm_rows(nvfp4v_ctx *ctx, const uint8_t *act, int64_t m, int64_t k, const void *packed,
                     int64_t n, float ts, float *c, hipStream_t stream);
// Row-major A of any m -> packed activations in blocks of CHUNK_M rows, both
// copies (act_packed_bytes(m, k) bytes).
int launch_pack_rows(nvfp4v_ctx *ctx, const uint16_t *a, int64_t m, int64_t k, uint8_t *act,
                     hipStream_t stream);
// Whether the GEMMs compute from the fp16 copy (NVFP4V_F16=0: from the bf16
// copy; both give the same C).
bool use_f16();
}  // namespace nvfp4v
