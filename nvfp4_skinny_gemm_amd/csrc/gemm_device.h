// Device code of the verify GEMM, shared by the per-call kernel (gemm.hip)
// and the persistent whole-pass kernel (pass.hip). See gemm.hip for the design.
#pragma once

#include <hip/hip_bf16.h>

#include "internal.h"

namespace nvfp4v {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int WG_WAVES = 4;
constexpr int WG_THREADS = 64 * WG_WAVES;
// A buffer offset past every range, so the load returns zeros. Every buffer
// resource here covers at most 0x7FFF0000 bytes (the host checks), and the
// largest constant or lane offset added to a base (< 32 KiB) keeps the sum
// below INT_MAX, so the offset arithmetic never overflows.
constexpr int OOB = 0x7FFF0000;
constexpr int RAW_BUFFER_FLAGS = 0x00020000;
// Cache policy of the weight loads: non-temporal. Each weight byte is read
// once per pass, so its lines are marked to leave the caches first and the
// packed activations, which every wave re-reads, stay resident (measured on
// MI355X: 2 % faster over the pass at 16 rows, 3.5 % at one row).
constexpr int WEIGHT_AUX = 2;
// s_getreg_b32 operand of HW_REG_XCC_ID (register 20, all 32 bits; bits 3:0
// hold the XCD the wave runs on).
constexpr int XCC_ID_HWREG = 0xF814;

// Work-group barrier that orders LDS only: waits for this wave's LDS
// operations but not for its global loads in flight (a fence before the
// barrier would wait for every outstanding load and empty the prefetch rings).
__device__ inline void lds_barrier_wg() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left open
  asm volatile("s_barrier" ::: "memory");
}

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

// The fp16 dequantisation: two E2M1 codes -> fp16 (unit scale), times the
// block scale as fp16 (ss: the scale in both halves) in one packed multiply.
// E4M3 scales are exact in fp16 (2^-9 is an fp16 normal), and so are their
// products with E2M1 values (at most 6 significant bits in [2^-10, 2688]):
// one VALU operation per weight against two for the bf16 form.
__device__ inline f16x8 dequant8h(uint32_t codes, f16x2 ss) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  const f16x8 r = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
  return r;
}

// A lane's dequantiser for one weight tile: its four block scales decoded
// once, then dequant(codes, i) for the 8 codes under scale i. F16 selects the
// fp16 form (fragments f16x8, v_mfma_f32_16x16x32_f16) over the bf16 form.
template <bool F16> struct Dq;
template <> struct Dq<false> {
  typedef bf16x8 frag;
  float s[4];
  Dq() = default;
  __device__ explicit Dq(uint32_t sw) { scales4(sw, s); }
  __device__ frag operator()(uint32_t codes, int i) const { return dequant8(codes, s[i]); }
};
template <> struct Dq<true> {
  typedef f16x8 frag;
  f16x2 s01, s23;
  Dq() = default;
  __device__ explicit Dq(uint32_t sw) {
    s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
    s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  }
  __device__ frag operator()(uint32_t codes, int i) const {
    // Whole-register selects and a broadcast shuffle (folded into the packed
    // multiply's operand selection) keep the scales in registers.
    const f16x2 p = (i >> 1) ? s23 : s01;
    return dequant8h(codes, (i & 1) ? __builtin_shufflevector(p, p, 1, 1) : __builtin_shufflevector(p, p, 0, 0));
  }
};

__device__ inline f32x4 mfma(const bf16x8 &w, const bf16x8 &a, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, a, c, 0, 0, 0);
}
__device__ inline f32x4 mfma(const f16x8 &w, const f16x8 &a, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(w, a, c, 0, 0, 0);
}

// The fp16 copy's value of a bf16 value: v * 2^ACT_F16_SHIFT as fp16 when
// exact, else the marker (internal.h).
__device__ inline uint16_t f16_act_bits(uint16_t bf) {
  // ldexp, not a multiply: the compiler fuses a multiply with the conversion
  // into v_fma_mix with a +0 addend, which turns -0 into +0.
  const float a = __uint_as_float((uint32_t)bf << 16);
  const _Float16 h = (_Float16)__builtin_ldexpf(a, ACT_F16_SHIFT);
  const bool exact = __builtin_ldexpf((float)h, -ACT_F16_SHIFT) == a;  // false for NaN
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return exact ? u : ACT_F16_MARK;
}

// End of a unit computed from the fp16 copy, in two steps around the
// work-group barrier that follows the sums' write to LDS. f16_flag (every
// wave, before the barrier): scales its sums back by 2^-ACT_F16_SHIFT (exact)
// and records in the wave's own LDS word whether any of them in a column
// below M is a NaN (every wave writes its word for every unit, so nothing
// needs clearing). Columns >= M are never stored, and the staged variants
// read whatever the buffer holds in those padding rows, so a NaN there must
// not send the unit to the bf16 path.
// f16_met_marker (after the barrier): whether any wave's sums held a NaN; the
// unit must then be computed again from the bf16 copy. The words are read
// before the next unit's barrier-separated writes.
__device__ inline unsigned *f16_flags() {
  static __shared__ unsigned s_f16bad[WG_WAVES];
  return s_f16bad;
}

template <int R, int MB>
__device__ inline void f16_flag(f32x4 (&acc)[R][MB], int M, int wave, int lane) {
  bool bad = false;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bool live = mb * 16 + (lane & 15) < M;  // this lane's column (row of A)
#pragma unroll
      for (int i = 0; i < 4; ++i) bad |= live && acc[r][mb][i] != acc[r][mb][i];
      acc[r][mb] *= 1.0f / (float)(1 << ACT_F16_SHIFT);
    }
  const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (lane == 0) f16_flags()[wave] = any ? 1u : 0u;
}

__device__ inline bool f16_met_marker() {
  const unsigned *f = f16_flags();
  unsigned x = 0;
#pragma unroll
  for (int w = 0; w < WG_WAVES; ++w) x |= f[w];
  return x != 0;
}

struct WTile {
  uint4 c[2];  // code halves
  uint32_t s;  // 4 scale bytes
};

// One row tile's k-tile (three loads per lane); `ok` false gives zeros.
__device__ inline void load_wtile(WTile &t, __amdgpu_buffer_rsrc_t rs, int kt, bool ok, int lane) {
  const int base = ok ? kt * TILE_BYTES : OOB;
  const auto c0 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + lane * 16, 0, WEIGHT_AUX);
  const auto c1 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + CODE_HALF_BYTES + lane * 16, 0, WEIGHT_AUX);
  const auto sc = __builtin_amdgcn_raw_buffer_load_b32(rs, base + SCALE_OFFSET + lane * 4, 0, WEIGHT_AUX);
  __builtin_memcpy(&t.c[0], &c0, 16);
  __builtin_memcpy(&t.c[1], &c1, 16);
  t.s = (uint32_t)sc;
}

// The 8 activation fragments of k-tile kt for each 16-row block (packed
// activations); lanes whose row is >= M, or `ok` false, read zeros.
template <int MB, class Frag>
__device__ inline void load_afrag(Frag (&b)[MB][8], __amdgpu_buffer_rsrc_t ra, int kt, bool ok,
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

// Code half C of a weight tile (dq: its dequantiser) into the MB
// accumulators: 4 x (dequant 8 codes, MB MFMAs).
template <int MB, int C, bool F16>
__device__ inline void compute_whalf(const WTile &t, const Dq<F16> &dq,
                                     const typename Dq<F16>::frag (&b)[MB][8], f32x4 (&acc)[MB]) {
  const uint32_t cw[4] = {t.c[C].x, t.c[C].y, t.c[C].z, t.c[C].w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const typename Dq<F16>::frag wf = dq(cw[j], 2 * C + (j >> 1));
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma(wf, b[mb][4 * C + j], acc[mb]);
  }
}

template <int MB, bool F16>
__device__ inline void compute_wtile(const WTile &t, const typename Dq<F16>::frag (&b)[MB][8],
                                     f32x4 (&acc)[MB]) {
  const Dq<F16> dq(t.s);
  compute_whalf<MB, 0, F16>(t, dq, b, acc);
  compute_whalf<MB, 1, F16>(t, dq, b, acc);
}

// compute_wtile followed by the tile's reload with k-tile kt, in two halves:
// the first code half and the scales are requested as soon as the first half
// has been consumed, the second code half after the second. The register
// variant's ring uses it (measured on MI355X: 2 % faster over the pass at
// 1-8 rows, 1.7 % at 16); the LDS variant keeps compute then load.
template <int MB, bool F16>
__device__ inline void compute_reload_wtile(WTile &t, const typename Dq<F16>::frag (&b)[MB][8],
                                            f32x4 (&acc)[MB], __amdgpu_buffer_rsrc_t rs, int kt, bool ok,
                                            int lane) {
  const Dq<F16> dq(t.s);
  const int base = ok ? kt * TILE_BYTES : OOB;
  compute_whalf<MB, 0, F16>(t, dq, b, acc);
  const auto c0 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + lane * 16, 0, WEIGHT_AUX);
  const auto sc = __builtin_amdgcn_raw_buffer_load_b32(rs, base + SCALE_OFFSET + lane * 4, 0, WEIGHT_AUX);
  __builtin_memcpy(&t.c[0], &c0, 16);
  t.s = (uint32_t)sc;
  compute_whalf<MB, 1, F16>(t, dq, b, acc);
  const auto c1 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + CODE_HALF_BYTES + lane * 16, 0, WEIGHT_AUX);
  __builtin_memcpy(&t.c[1], &c1, 16);
}

// Occupancy target (waves per SIMD) for the register allocator: three when
// the ring (D k-tiles of R weight tiles and MB fragment blocks), the
// accumulators and ~40 working registers fit in 168 VGPRs, else two.
template <int MB, int R, int D, bool A2 = false>
constexpr int waves_per_simd() {
  return ((A2 ? R * 9 + 2 * MB * 32 : D * (R * 9 + MB * 32)) + R * MB * 4 + 40) <= 168 ? 3 : 2;
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
// GEMM's packed activations (both copies) and the optional row-major copies.
__device__ inline void store_next(const Epilogue &epi, int mblocks, int m, int j, int cols,
                                  const float (&o)[4]) {
  uint16_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = bf16_bits(o[i]);
  const uint32_t lo = (uint32_t)b[0] | ((uint32_t)b[1] << 16);
  const uint32_t hi = (uint32_t)b[2] | ((uint32_t)b[3] << 16);
  const uint2 v = make_uint2(lo, hi);
  // Write-through (system-coherent) stores: a consumer on another die reads
  // them through its own L2 without a write-back fence.
  uint8_t *dst = epi.act + act_offset(m, j, mblocks);
  __hip_atomic_store(reinterpret_cast<uint64_t *>(dst), (uint64_t)lo | ((uint64_t)hi << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_SYSTEM);
  if (epi.act16) {
    const uint64_t h = (uint64_t)f16_act_bits(b[0]) | ((uint64_t)f16_act_bits(b[1]) << 16) |
                       ((uint64_t)f16_act_bits(b[2]) << 32) | ((uint64_t)f16_act_bits(b[3]) << 48);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(dst + epi.act16), h, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (epi.rm0) *reinterpret_cast<uint2 *>(epi.rm0 + (size_t)m * cols + j) = v;
  if (epi.rm1) *reinterpret_cast<uint2 *>(epi.rm1 + (size_t)m * cols + j) = v;
}

// One lane's final values of row tile rt and 16-row block mb (lane l holds
// D[n = 16 rt + 4 (l / 16) + i][m = 16 mb + l % 16], i = 0..3): times ts,
// into C and, for EPI_SCALE, into the next GEMM's activations. MB is the
// number of 16-row blocks of the activations (the next GEMM's too).
template <int MB>
__device__ inline void epi_tile_lane(f32x4 v, int rt, int mb, int lane, int M, int N, int nrt, float ts,
                                     float *C, const Epilogue &epi) {
  const int m = mb * 16 + (lane & 15);
  const int n0 = rt * ROWS_PER_TILE + 4 * (lane >> 4);
  if (m >= M || rt >= nrt || n0 >= N) return;
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

// The same for a (gate, up) pair of row tiles rtg (even) and rtg + 1 (EPI_PAIR):
// C in natural [gate | up] order and the glue sum into the next activations.
template <int MB>
__device__ inline void epi_pair_lane(f32x4 vg, f32x4 vu, int rtg, int mb, int lane, int M, int N, int nrt,
                                     float ts, float *C, const Epilogue &epi) {
  const int half = N / 2;
  const int m = mb * 16 + (lane & 15);
  if (m >= M || rtg + 1 >= nrt) return;
  const int j0 = (rtg / 2) * ROWS_PER_TILE + 4 * (lane >> 4);
  if (j0 >= half) return;
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

// Final values of the work-group's tiles are red[w][r][mb][l] summed over the
// first nw slots (wave order). Writes C (times ts) and the fused glue.
template <int MB, int R>
__device__ inline void epilogue(const f32x4 *red, int nw, int tid, int M, int N, int nrt, int rt0,
                                float ts, float *C, const Epilogue &epi) {
  if (epi.mode == EPI_PAIR) {
    for (int it = tid; it < (R / 2) * MB * 64; it += WG_THREADS) {
      const int p = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      f32x4 vg = red[((0 * R + 2 * p) * MB + mb) * 64 + l];
      f32x4 vu = red[((0 * R + 2 * p + 1) * MB + mb) * 64 + l];
      for (int wv = 1; wv < nw; ++wv) {
        vg += red[((wv * R + 2 * p) * MB + mb) * 64 + l];
        vu += red[((wv * R + 2 * p + 1) * MB + mb) * 64 + l];
      }
      epi_pair_lane<MB>(vg, vu, rt0 + 2 * p, mb, l, M, N, nrt, ts, C, epi);
    }
    return;
  }
  for (int it = tid; it < R * MB * 64; it += WG_THREADS) {
    const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
    f32x4 v = red[((0 * R + r) * MB + mb) * 64 + l];
    for (int wv = 1; wv < nw; ++wv) v += red[((wv * R + r) * MB + mb) * 64 + l];
    epi_tile_lane<MB>(v, rt0 + r, mb, l, M, N, nrt, ts, C, epi);
  }
}

// Arguments of one GEMM (one phase of the pass, or one verify_gemm call).
struct GemmArgs {
  const uint8_t *act;  // packed activations (the bf16 copy)
  int M, act_bytes;    // act_bytes: one copy
  // > 0: the fp16 copy lies act16 bytes after `act`, and the units compute
  // from it (computing a unit again from the bf16 copy where it meets a
  // marker); 0: from the bf16 copy.
  int act16 = 0;
  // M > 64 (the wide unit only): the rows come as two packed blocks, rows
  // 0..63 at `act` and rows 64.. at act + act_blk1 bytes (the layout
  // pack_activations writes for more than 64 rows).
  int act_blk1 = 0;
  const uint8_t *W;  // packed weights
  int N, nrt, nkt, kts_per_split, ksplit;
  float ts;
  float *C, *part;
  unsigned *counters;
  Epilogue epi;
  // Row blocks of the launch. The grid's x may be padded past it (to a
  // multiple of 8 for the exchange below); padding work-groups do nothing.
  int nrb = 0x7FFFFFFF;
  // Split-K exchange through the L2 of one XCD (unit_tail): set when the grid's
  // x is a multiple of 8, so that the pieces of a row block have linear ids
  // congruent mod 8, and the dispatch probe found such ids on one XCD. The
  // row blocks begun and completed are then counted in `status` (below).
  int xcd_local = 0;
  unsigned *status = nullptr;
};

// Row-block counts of the exchange through one XCD's L2, in the context's
// status lines: line x (DEV_LINE_WORDS words) counts, for work-groups on XCD
// x, the row blocks begun (by their piece 0) and completed (by their last
// arriver). A row block whose pieces ran on two XCDs took its tickets in two
// L2s, so none of its pieces saw the last ticket: it is begun and never
// completed, and the host reports the difference. Fire-and-forget atomics, off
// the exchange's critical path.
__device__ inline void count_row_block(unsigned *status, int which) {
  const unsigned x = (unsigned)__builtin_amdgcn_s_getreg(XCC_ID_HWREG) & 7u;
  __hip_atomic_fetch_add(status + x * DEV_LINE_WORDS + which, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// A unit that computed from the fp16 copy and met a marker (called between
// its fp16 and bf16 runs): counted in the context's status lines, if any.
__device__ inline void count_f16_redone(const GemmArgs &g) {
  if (g.act16 && g.status && threadIdx.x == 0) count_row_block(g.status, DEV_F16_REDONE);
}

// End of a work unit whose RT row tiles' sums sit in LDS: red[((w * RT + r) *
// MB + mb) * 64 + lane] for slices w < NW (summed in slice order). The unit is
// piece `ks` of the `ksplit` pieces (consecutive k-ranges, in k order) its row
// block is cut into. With one piece the epilogue runs here; otherwise the unit
// publishes its partial tile sums, takes a ticket, and the last of the row
// block's pieces to arrive sums them in piece order 0..ksplit-1 and runs the
// epilogue. The exchange meets either in memory (system-scope stores, ticket
// and loads, which bypass the dies' L2s) or, with g.xcd_local, in the L2 of
// the one XCD that runs all pieces of the row block: plain stores (the vector
// L1 writes through to the L2), a ticket atomic executed in that L2, and loads
// that read through to it. Each row block's partial lines are read once per
// launch, by its last arriver, so no L1 can hold a stale copy of them. The
// ticket slot follows the NW * RT * MB * 64 sums in LDS. Every thread of the
// work-group calls this; it returns with the LDS free.
template <int MB, int RT, int NW, bool REDUCER = false>
__device__ inline void unit_tail(const GemmArgs &g, int rb, int ks, int ksplit, f32x4 *red, int tid) {
  const int M = g.M, N = g.N, nrt = g.nrt;
  float *__restrict__ part = g.part;
  unsigned *__restrict__ counters = g.counters;
  const int rt0 = rb * RT;
  const int npad = nrt * ROWS_PER_TILE;
  constexpr int ITEMS = RT * MB * 64;
  int nw = NW;
  if (REDUCER && ksplit > 1 && g.xcd_local) {
    // Designated reducer (exchange through one XCD's L2 only): the row
    // block's last piece, which has the highest linear id and is dispatched
    // after its siblings, keeps its own partial in LDS and waits for the
    // others to publish theirs, instead of every piece publishing and the last
    // to arrive reducing. The siblings never wait on anything, and they were
    // dispatched before the reducer, so the wait ends; a 1 s bound on the
    // 100 MHz clock makes any other outcome an unfinished row block, which the
    // begun/completed counts report. Their tickets use the low 16 bits; the
    // reducer polls with an atomic add in the high bits (an atomic executes in
    // the L2; a plain load could keep hitting a stale L1 line) and then
    // clears the word. The sum keeps the split order 0..ksplit-1.
    unsigned *s_flag = reinterpret_cast<unsigned *>(red + NW * RT * MB * 64);
    if (ks != ksplit - 1) {
      for (int it = tid; it < ITEMS; it += WG_THREADS) {
        const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
        f32x4 v = red[((0 * RT + r) * MB + mb) * 64 + l];
#pragma unroll
        for (int wv = 1; wv < NW; ++wv) v += red[((wv * RT + r) * MB + mb) * 64 + l];
        const int m = mb * 16 + (l & 15), rt = rt0 + r;
        if (m >= M || rt >= nrt) continue;
        *reinterpret_cast<f32x4 *>(part + ((size_t)ks * M + m) * npad + rt * ROWS_PER_TILE + 4 * (l >> 4)) = v;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) (void)__hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return;
    }
    if (tid == 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      unsigned n = 0;
      while (((n = __hip_atomic_fetch_add(&counters[rb], 0x10000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) &
              0xFFFFu) < (unsigned)(ksplit - 1)) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > 100000000ull) break;
        __builtin_amdgcn_s_sleep(1);
      }
      const bool ok = (n & 0xFFFFu) == (unsigned)(ksplit - 1);
      *s_flag = ok ? 1u : 0u;
      if (ok) {
        __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        count_row_block(g.status, DEV_ROWS_DONE);
      }
    }
    __syncthreads();
    if (!*s_flag) return;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void *)part, (short)0, (int)((size_t)ksplit * M * npad * sizeof(float)), RAW_BUFFER_FLAGS);
    for (int it = tid; it < ITEMS; it += WG_THREADS) {
      const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      f32x4 own = red[((0 * RT + r) * MB + mb) * 64 + l];
#pragma unroll
      for (int wv = 1; wv < NW; ++wv) own += red[((wv * RT + r) * MB + mb) * 64 + l];
      const int m = mb * 16 + (l & 15), rt = rt0 + r;
      f32x4 v = own;
      if (m < M && rt < nrt) {
        const size_t off = (size_t)m * npad + rt * ROWS_PER_TILE + 4 * (l >> 4);
        for (int s2 = 0; s2 < ksplit - 1; ++s2) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b128(rp, (int)((off + (size_t)s2 * M * npad) * sizeof(float)), 0, 1);
          f32x4 y;
          __builtin_memcpy(&y, &x, 16);
          v = s2 == 0 ? y : v + y;
        }
        v += own;
      }
      red[((0 * RT + r) * MB + mb) * 64 + l] = v;
    }
    __syncthreads();
    nw = 1;
  } else if (ksplit > 1) {
    const bool local = g.xcd_local != 0;
    for (int it = tid; it < ITEMS; it += WG_THREADS) {
      const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      f32x4 v = red[((0 * RT + r) * MB + mb) * 64 + l];
#pragma unroll
      for (int wv = 1; wv < NW; ++wv) v += red[((wv * RT + r) * MB + mb) * 64 + l];
      const int m = mb * 16 + (l & 15), rt = rt0 + r;
      if (m >= M || rt >= nrt) continue;
      float *dst = part + ((size_t)ks * M + m) * npad + rt * ROWS_PER_TILE + 4 * (l >> 4);
      if (local) {
        *reinterpret_cast<f32x4 *>(dst) = v;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(dst + i, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    // The partial stores are acknowledged (by the L2, or by memory) once this
    // wave's counter drains; the clobber keeps the compiler from moving them
    // below the wait.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    unsigned *s_ticket = reinterpret_cast<unsigned *>(red + NW * RT * MB * 64);
    if (tid == 0)
      *s_ticket = local ? __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)
                        : __hip_atomic_fetch_add(&counters[rb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    const bool last = *s_ticket == (unsigned)(ksplit - 1);
    __syncthreads();  // everyone has read the ticket before the slot is reused
    if (!last) return;
    if (local && tid == 0) count_row_block(g.status, DEV_ROWS_DONE);
    // Last to arrive: sum the splits in order 0..ksplit-1 into slice 0.
    // (Buffer loads with sc0 read through the L1; every offset lies inside the
    // ksplit * M * npad floats of the partials.)
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void *)part, (short)0, (int)((size_t)ksplit * M * npad * sizeof(float)), RAW_BUFFER_FLAGS);
    for (int it = tid; it < ITEMS; it += WG_THREADS) {
      const int r = it / (MB * 64), mb = (it / 64) % MB, l = it & 63;
      const int m = mb * 16 + (l & 15), rt = rt0 + r;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m < M && rt < nrt) {
        const size_t off = (size_t)m * npad + rt * ROWS_PER_TILE + 4 * (l >> 4);
        if (local) {
          for (int s2 = 0; s2 < ksplit; ++s2) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rp, (int)((off + (size_t)s2 * M * npad) * sizeof(float)), 0, 1);
            f32x4 y;
            __builtin_memcpy(&y, &x, 16);
            v = s2 == 0 ? y : v + y;
          }
        } else {
          const float *src = part + off;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          for (int s2 = 1; s2 < ksplit; ++s2) {
            const float *s2p = src + (size_t)s2 * M * npad;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              v[i] += __hip_atomic_load(s2p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          }
        }
      }
      red[((0 * RT + r) * MB + mb) * 64 + l] = v;
    }
    __syncthreads();
    if (tid == 0) {
      if (local) __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      else __hip_atomic_store(&counters[rb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    nw = 1;
  }
  epilogue<MB, RT>(red, nw, tid, M, N, nrt, rt0, g.ts, g.C, g.epi);
  __syncthreads();  // LDS free for the next unit
}

// One work unit: row block `rb` (R row tiles) x k-tiles [kA, kB), piece `ks`
// of the row block's `ksplit` pieces, by the whole work-group; its 4 waves
// split the unit's k-tiles. D is the depth of each
// wave's ring of k-tiles in flight (D = 1 at large M, where two copies of the
// activation fragments do not fit in registers; 3 or 4 for short units, where
// latency, not throughput, bounds the unit). `red` is the work-group's LDS
// buffer of WG_WAVES * R * MB * 64 f32x4. Every thread of the work-group calls
// this with the same arguments; it returns with the LDS buffer free for the
// next unit. F16: computes from the fp16 copy and returns false, before the
// exchange and with nothing written, if the unit met a marker (the caller
// then runs the unit with F16 false); else returns true.
template <int MB, int R, int D, bool A2, bool F16>
__device__ inline bool gemm_unit(const GemmArgs &g, int rb, int kA, int kB, int ks, int ksplit, f32x4 *red) {
  typedef typename Dq<F16>::frag Frag;
  const uint8_t *__restrict__ act = g.act + (F16 ? g.act16 : 0);
  const int M = g.M, act_bytes = g.act_bytes, nrt = g.nrt, nkt = g.nkt;
  const uint8_t *__restrict__ W = g.W;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int rt0 = rb * R;
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

  if constexpr (A2) {
    // One-deep weight ring (each tile reloaded in halves while it is
    // consumed) with the activation fragments two deep: k-tile i + 1's
    // fragments are requested before k-tile i is computed, so their L2
    // latency hides behind a whole k-tile of work instead of stalling the
    // next one. For MB x R where two full rings do not fit in registers.
    static_assert(D == 1, "the two-deep activation ring goes with a one-deep weight ring");
    WTile w[R];
    Frag a[2][MB][8];
    load_afrag<MB>(a[0], ra, kbeg, 0 < n, M, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) load_wtile(w[r], rs[r], kbeg, 0 < n, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_afrag<MB>(a[1], ra, kbeg + 1, 1 < n, M, lane);
    __builtin_amdgcn_sched_barrier(0);
    // Step d of iteration i computes k-tile i + d from (w, a[d]), reloading w
    // with k-tile i + d + 1 and then a[d] with k-tile i + d + 2; every step
    // issues the same loads in the same order (zeros past the range).
    int i = 0;
    for (; i + 2 <= n; i += 2) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          compute_reload_wtile<MB, F16>(w[r], a[d], acc[r], rs[r], kbeg + i + d + 1, i + d + 1 < n, lane);
        load_afrag<MB>(a[d], ra, kbeg + i + d + 2, i + d + 2 < n, M, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (i < n) {
#pragma unroll
      for (int r = 0; r < R; ++r) compute_wtile<MB, F16>(w[r], a[0], acc[r]);
    }
    if (F16) f16_flag(acc, g.M, wave, lane);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
    __syncthreads();
    if (F16 && f16_met_marker()) return false;
    unit_tail<MB, R, WG_WAVES>(g, rb, ks, ksplit, red, tid);
    return true;
  }

  // A ring of D k-tiles (weights and activation fragments) per wave: slot d
  // holds k-tiles kbeg + d, kbeg + d + D, ...; each slot is refilled D
  // k-tiles ahead right after it is consumed. The loop body consumes all D
  // slots and issues the same loads in the same order every time (loads past
  // the wave's range use an offset that returns zeros), with scheduling
  // barriers keeping each refill in place, so the compiler's wait counts leave
  // D - 1 k-tiles in flight. The remaining k-tiles (fewer than D) are
  // computed after the loop without new loads.
  WTile w[D][R];
  Frag a[D][MB][8];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_afrag<MB>(a[d], ra, kbeg + d, d < n, M, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) load_wtile(w[d][r], rs[r], kbeg + d, d < n, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  int i = 0;
  for (; i + D <= n; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        compute_reload_wtile<MB, F16>(w[d][r], a[d], acc[r], rs[r], kbeg + i + d + D, i + d + D < n, lane);
      load_afrag<MB>(a[d], ra, kbeg + i + d + D, i + d + D < n, M, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    if (i + d < n) {
#pragma unroll
      for (int r = 0; r < R; ++r) compute_wtile<MB, F16>(w[d][r], a[d], acc[r]);
    }
  }
  if (F16) f16_flag(acc, g.M, wave, lane);

  // Sum the 4 waves' tiles in wave order (LDS), then either finish here
  // (ksplit == 1) or exchange partial tiles with the other splits.
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
  __syncthreads();
  if (F16 && f16_met_marker()) return false;
  unit_tail<MB, R, WG_WAVES>(g, rb, ks, ksplit, red, tid);
  return true;
}


// The same GEMM with the activations staged in LDS once per work-group:
// the 4 waves split N (wave w owns row tiles rt0 + w R .. + R - 1, RT = 4 R
// per unit) and walk the same k-tiles in lockstep. Per k-tile i every thread
// loads MB x 32 bytes of the packed activations (the work-group's copy) two
// k-tiles ahead into registers and writes them to a two-slot LDS ring one
// k-tile ahead; each wave reads its MFMA fragments from LDS and reuses them
// across its R weight tiles. Weights stream through each wave's two-deep
// register ring as in gemm_unit. One work-group barrier per k-tile.
// `lds` holds 2 slots of MB * 8 KiB, then the RT tiles' sums and the ticket.
// F16 and the result as in gemm_unit.
template <int MB, int R, bool F16>
__device__ inline bool gemm_unit_lds(const GemmArgs &g, int rb, int ks, uint8_t *lds) {
  typedef typename Dq<F16>::frag Frag;
  constexpr int RT = WG_WAVES * R;
  constexpr int SLOT = MB * 8 * ACT_FRAG_BYTES;  // one k-tile of packed activations
  constexpr int PER_THREAD = SLOT / WG_THREADS / 16;  // 16-byte chunks per thread (2 MB)
  const int nrt = g.nrt, nkt = g.nkt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt0 = rb * RT + wave * R;
  const int kA = ks * g.kts_per_split;
  const int n = min(nkt, kA + g.kts_per_split) - kA;  // k-tiles of the unit (>= 1)
  const int stripe_bytes = nkt * TILE_BYTES;
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    const uint8_t *base = g.W + (size_t)min(rt, nrt - 1) * (size_t)stripe_bytes;
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, rt < nrt ? stripe_bytes : 0,
                                              RAW_BUFFER_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(g.act + (F16 ? g.act16 : 0)), (short)0, g.act_bytes, RAW_BUFFER_FLAGS);
  f32x4 *red = reinterpret_cast<f32x4 *>(lds + 2 * SLOT);

  // Staging: k-tile j's packed block is contiguous (SLOT bytes at j * SLOT);
  // thread t moves chunks x = t, t + 256, ... of it. Chunk x holds row
  // 16 (x >> 9) + (x & 15) (fragment x >> 6, lane x & 63). With one row block
  // a row >= M gets an offset of OOB, so its loads return zeros without a
  // memory access (at M = 1 that skips 15 of every 16); with more, at most
  // 15 of 32 or more rows are padding and every chunk is loaded (rows >= M
  // then hold whatever the buffer holds; the marker test ignores them).
  // Offsets are unsigned 32-bit: the largest, OOB + OOB, does not wrap.
  uint32_t lo[PER_THREAD];
#pragma unroll
  for (int c = 0; c < PER_THREAD; ++c) {
    const int x = c * WG_THREADS + tid;
    lo[c] = MB > 1 || (x & 15) < g.M ? (uint32_t)x * 16 : (uint32_t)OOB;
  }
  auto stage_load = [&](uint4 (&v)[PER_THREAD], int j) {
    const uint32_t base = j < n ? (uint32_t)((kA + j) * SLOT) : (uint32_t)OOB;
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) {
      const auto y = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(base + lo[c]), 0, 0);
      __builtin_memcpy(&v[c], &y, 16);
    }
  };
  auto stage_store = [&](const uint4 (&v)[PER_THREAD], int slot) {
    uint4 *dst = reinterpret_cast<uint4 *>(lds + slot * SLOT);
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) dst[c * WG_THREADS + tid] = v[c];
  };
  auto frags = [&](Frag (&b)[MB][8], int slot) {
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

  WTile w0[R], w1[R];
  uint4 s0[PER_THREAD], s1[PER_THREAD];
  stage_load(s0, 0);
#pragma unroll
  for (int r = 0; r < R; ++r) load_wtile(w0[r], rs[r], kA, true, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(s1, 1);
#pragma unroll
  for (int r = 0; r < R; ++r) load_wtile(w1[r], rs[r], kA + 1, n > 1, lane);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(s0, 0);
  stage_load(s0, 2);
  __builtin_amdgcn_sched_barrier(0);

  // Iteration i: barrier (slot i%2 holds k-tile i; slot (i+1)%2 is free),
  // fragments of k-tile i, stage k-tile i+1 into LDS and request k-tile i+3's
  // activations (before the compute: 0.8 % faster over the pass at 12-16
  // rows), compute, then request k-tile i+2's weights into the registers the
  // compute has just freed.
#define NVFP4V_LDS_STEP(W, S_NEXT, SLOT_I)                                               \
  {                                                                                               \
    lds_barrier_wg();                                                                             \
    Frag b[MB][8];                                                                                \
    frags(b, SLOT_I);                                                                             \
    stage_store(S_NEXT, 1 - SLOT_I);                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    stage_load(S_NEXT, i + 3);                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    _Pragma("unroll") for (int r = 0; r < R; ++r) compute_wtile<MB, F16>(W[r], b, acc[r]);       \
    __builtin_amdgcn_sched_barrier(0);                                                            \
    _Pragma("unroll") for (int r = 0; r < R; ++r) load_wtile(W[r], rs[r], kA + i + 2, i + 2 < n, lane); \
    __builtin_amdgcn_sched_barrier(0);                                                            \
  }
  int i = 0;
  for (; i + 1 < n; i += 2) {
    NVFP4V_LDS_STEP(w0, s1, 0)
    ++i;
    NVFP4V_LDS_STEP(w1, s0, 1)
    --i;
  }
  if (i < n) NVFP4V_LDS_STEP(w0, s1, 0)
#undef NVFP4V_LDS_STEP

  // Each wave's tiles into slice 0 of the sums (tile wave * R + r), then the
  // shared tail (split-K exchange, epilogue).
  if (F16) f16_flag(acc, g.M, wave, lane);
  lds_barrier_wg();
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
  __syncthreads();
  if (F16 && f16_met_marker()) return false;
  unit_tail<MB, RT, 1, true>(g, rb, ks, g.ksplit, red, tid);
  return true;
}

// The wide-M unit (33..128 rows): like gemm_unit_lds, the 4 waves split N
// (wave w owns R of the work-group's 4R row tiles) and walk the same k-tiles,
// with each k-tile's packed activations (MB x 8 KiB) staged once per
// work-group into LDS. The difference is the order of the products: per group
// of 8 codes, a wave dequantises its R row tiles once and then runs them
// against every 16-row block's fragment, read from LDS one at a time. A
// fragment is reused across R row tiles and a dequantised weight across MB
// blocks, so neither the fragments of all MB blocks (MB x 32 VGPRs) nor a
// second dequant is needed. One LDS slot: the next k-tile's activations wait
// in registers (MB / 2 16-byte chunks per thread) until every wave has
// finished reading the slot; two work-group barriers per k-tile.
template <int MB, int R, bool F16>
__device__ inline bool gemm_unit_wide(const GemmArgs &g, int rb, int ks, uint8_t *lds) {
  typedef typename Dq<F16>::frag Frag;
  constexpr int RT = WG_WAVES * R;
  constexpr int SLOT = MB * 8 * ACT_FRAG_BYTES;       // one k-tile of packed activations
  constexpr int PER_THREAD = SLOT / WG_THREADS / 16;  // 16-byte chunks per thread
  static_assert(SLOT % (WG_THREADS * 16) == 0, "staging split");
  const int nrt = g.nrt, nkt = g.nkt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt0 = rb * RT + wave * R;
  const int kA = ks * g.kts_per_split;
  const int n = min(nkt, kA + g.kts_per_split) - kA;  // k-tiles of the unit (>= 1)
  const int stripe_bytes = nkt * TILE_BYTES;
  __amdgpu_buffer_rsrc_t rs[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    const uint8_t *base = g.W + (size_t)min(rt, nrt - 1) * (size_t)stripe_bytes;
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, rt < nrt ? stripe_bytes : 0,
                                              RAW_BUFFER_FLAGS);
  }
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(g.act + (F16 ? g.act16 : 0)), (short)0, g.act_bytes, RAW_BUFFER_FLAGS);

  // The slot holds [row block][fragment q][lane]; thread t moves chunks
  // c * 256 + t, i.e. row block c / 2, second half of its fragments if c is
  // odd. Row blocks 0..3 come from the first packed block of 64 rows (B0 of
  // them per k-tile), the rest from the second (MB - 4 per k-tile).
  constexpr int B0 = MB < 4 ? MB : 4;
  uint4 stage[PER_THREAD];
  auto stage_load = [&](int j) {
    const int kt = kA + j;
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) {
      const int mb = c / 2;
      const int off = mb < B0 ? (kt * B0 + mb) * 8 * ACT_FRAG_BYTES
                              : g.act_blk1 + (kt * (MB - B0) + (mb - B0)) * 8 * ACT_FRAG_BYTES;
      const int base = j < n ? off + ((c & 1) * WG_THREADS + tid) * 16 : OOB;
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(ra, base, 0, 0);
      __builtin_memcpy(&stage[c], &x, 16);
    }
  };
  auto stage_store = [&]() {
    uint4 *dst = reinterpret_cast<uint4 *>(lds);
#pragma unroll
    for (int c = 0; c < PER_THREAD; ++c) dst[c * WG_THREADS + tid] = stage[c];
  };
  const uint4 *afr = reinterpret_cast<const uint4 *>(lds);

  f32x4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Products of one k-tile: for each half C and group j of 8 codes, R
  // dequantised weight fragments against MB activation fragments.
  auto compute = [&](const WTile (&W)[R]) {
    Dq<F16> dq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dq[r] = Dq<F16>(W[r].s);
#pragma unroll
    for (int C = 0; C < 2; ++C)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Frag wf[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t cw = j == 0 ? W[r].c[C].x : j == 1 ? W[r].c[C].y : j == 2 ? W[r].c[C].z : W[r].c[C].w;
          wf[r] = dq[r](cw, 2 * C + (j >> 1));
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint4 x = afr[(mb * 8 + 4 * C + j) * 64 + lane];
          Frag b;
          __builtin_memcpy(&b, &x, 16);
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r][mb] = mfma(wf[r], b, acc[r][mb]);
        }
      }
  };

  WTile w0[R], w1[R];
  stage_load(0);
#pragma unroll
  for (int r = 0; r < R; ++r) load_wtile(w0[r], rs[r], kA, true, lane);
#pragma unroll
  for (int r = 0; r < R; ++r) load_wtile(w1[r], rs[r], kA + 1, n > 1, lane);
  __builtin_amdgcn_sched_barrier(0);

  // Iteration i: every wave has finished reading k-tile i - 1 (barrier), the
  // slot takes k-tile i from the staging registers, which then request
  // k-tile i + 1; after a second barrier the slot is read; the weights of
  // k-tile i + 2 go into the ring registers the products have just freed.
#define NVFP4V_WIDE_STEP(W)                                                                         \
  {                                                                                                 \
    __syncthreads();                                                                                \
    stage_store();                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                              \
    stage_load(i + 1);                                                                              \
    __builtin_amdgcn_sched_barrier(0);                                                              \
    lds_barrier_wg();                                                                               \
    compute(W);                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                              \
    _Pragma("unroll") for (int r = 0; r < R; ++r) load_wtile(W[r], rs[r], kA + i + 2, i + 2 < n, lane); \
    __builtin_amdgcn_sched_barrier(0);                                                              \
  }
  int i = 0;
  for (; i + 1 < n; i += 2) {
    NVFP4V_WIDE_STEP(w0)
    ++i;
    NVFP4V_WIDE_STEP(w1)
    --i;
  }
  if (i < n) NVFP4V_WIDE_STEP(w0)
#undef NVFP4V_WIDE_STEP

  // The tiles' sums reuse the LDS (slice 0, tile wave * R + r), then the
  // shared tail (split-K exchange, epilogue).
  f32x4 *red = reinterpret_cast<f32x4 *>(lds);
  if (F16) f16_flag(acc, g.M, wave, lane);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
  __syncthreads();
  if (F16 && f16_met_marker()) return false;
  unit_tail<MB, RT, 1, true>(g, rb, ks, g.ksplit, red, tid);
  return true;
}

}  // namespace dev
}  // namespace nvfp4v
