// The verify pass in stream mode: one cooperatively launched kernel per 32
// layers in which HBM keeps streaming weights across GEMM boundaries.
//
// A verify pass reads 0.5625 bytes per weight and almost nothing else
// (TandemLLM manual, "What TandemLLM is", 1.2 "Two levers": a pass over 16
// tree rows reads the same weights as one over a single row), so its time is
// set by how steadily HBM is kept busy. Its GEMMs depend on each other only
// through their small activations, never through the weights, so the next
// GEMM's weights can be on their way while the previous GEMM finishes.
//
// Work split. Every GEMM (one projection of one layer: a "phase") is cut into
// one rectangle per work-group: the grid's G work-groups form G / gk row
// groups of R row tiles, each cut along K into gk k-groups of S k-tiles, so
// every work-group streams the same bytes in every phase (for the dense stack
// of 5120 / 17408: 75, 25, 170 and 85 tiles per work-group for q|k|v, o,
// gate|up and down, with gk = 4). A work-group takes its place from the XCD it
// runs on (the hardware register) and an arrival count per XCD, and the gk
// work-groups of a row group are places on one XCD, so their split-K partial
// sums meet in that XCD's L2 by construction.
//
// Roles in a work-group (6 waves, one work-group per CU):
//  * wave 4 streams the work-group's weight tiles, phase after phase, from HBM
//    straight into a 48-slot LDS ring (buffer_load ... lds: no VGPRs), up to 20
//    tiles in flight. It waits only for a free slot, never for another
//    work-group, so while the consumers sit at a phase boundary the next
//    phase's weights keep arriving (the ring holds about 4 us of streaming).
//  * wave 5 loads each k-tile of packed activations into a small LDS ring,
//    once per work-group, and runs the grid barrier between phases (the next
//    phase's activations are written by every row group's epilogue).
//  * waves 0..3 consume: per k-tile they read the activation fragments from
//    LDS once and, for each weight tile of theirs, read it from the ring,
//    dequantise it in registers and run the MFMAs (the per-call GEMM's
//    compute_wtile). Wave w owns every fourth unit of the rectangle's rows (a
//    unit is a row tile, or a (gate, up) pair of row tiles); the 0..3 units
//    left over are dealt out k-tile by k-tile, so the four waves get equal
//    work in every phase.
//
// Reduction, in a fixed order. The row group's k-group p % gk reduces phase p
// (the role rotates). Every other k-group publishes its waves' partial tiles
// in the XCD's L2 and counts them in per-wave tickets; the reducer's wave w
// sums the gk partials of its own units in k-group order and runs the fused
// epilogue (the glue into the next phase's packed activations). Leftover
// units are summed over k-groups and waves, in that order, by one reducer
// wave each. Every sum keeps its order, so the pass is bitwise reproducible.
//
// Coherence across the dies' L2 caches is as in the other persistent kernels:
// epilogues write the next activations with system-coherent stores, each phase
// reads a buffer no other phase of the launch uses, and every wait is bounded
// (2 s on the 100 MHz clock), after which an error flag is set and every wave
// leaves, so a broken launch cannot hang the GPU.
#include <hip/hip_bf16.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdlib>

#include "pass_common.h"

using namespace nvfp4v;
using namespace nvfp4v::dev;
using namespace nvfp4v::passk;

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int SC = 4;                 // consumer waves
constexpr int SW_THREADS = (SC + 2) * 64;
constexpr int OWN_SLOTS = 8;          // row tiles a consumer wave owns in a phase
constexpr int EXTRA_SLOTS = 4;        // rows of the leftover units
constexpr int SLOTS = OWN_SLOTS + EXTRA_SLOTS;
constexpr int NSLOT = 48;             // weight ring slots (one tile each)
constexpr int WLAG = 20;              // weight tiles in flight (3 loads each; vmcnt <= 63)

// Context counter words used by this mode (all zero between passes).
constexpr int XCD_CNT = 0;    // [16 x]: places taken on XCD x (x = 0..7)
constexpr int XCD_IDS = 8;    // [XCD_IDS + 16 x]: 1 + the hardware id of the XCD that is x
constexpr int RG_CNT = 128;  // [RG_CNT + 8 rg + i]: row group rg's tickets: own-unit partials
                             // for consumer wave i < 4, leftover partials (4) and their readers (5)
constexpr int MAX_ROW_GROUPS = 256;
constexpr int STREAM_COUNTER_WORDS = RG_CNT + 8 * MAX_ROW_GROUPS;

template <int MB>
constexpr int n_act_slots() { return MB == 1 ? 4 : 3; }
template <int MB>
constexpr int act_slot_bytes() { return MB * 8 * ACT_FRAG_BYTES; }

// LDS flag words after the rings: tiles published by the weight wave, k-tiles
// of activations published by the activation wave, consumer phase completions,
// an abort flag, each consumer's activation progress, and per ring slot the
// number of times it has been consumed.
constexpr int F_WPUB = 0, F_APUB = 1, F_DONE = 2, F_ABORT = 3, F_APROG = 4, F_CONS = 8,
              F_WORDS = F_CONS + NSLOT;

template <int MB>
constexpr size_t stream_lds_bytes() {
  return (size_t)NSLOT * TILE_BYTES + (size_t)n_act_slots<MB>() * act_slot_bytes<MB>() + F_WORDS * 4;
}

// LDS flag accesses are written out so that the compiler's wait-count pass does
// not take them for reads of the LDS the DMA loads are filling (it would wait
// for every load in flight before each one). One lane writes.
__device__ inline uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }
__device__ inline unsigned lds_ld(const unsigned *p) {
  unsigned v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ inline void lds_st(unsigned *p, unsigned v, int lane) {
  if (lane == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ inline void lds_inc(unsigned *p, int lane) {
  if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(p)), "v"(1u) : "memory");
}

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Where a pass gave up (the error word keeps the first site; the pass reports
// NVFP4V_E_TIMEOUT and nvfp4v_pass_error_site the site).
constexpr unsigned SITE_PLACE = 16, SITE_WEIGHT_SLOT = 17, SITE_ACT_SLOT = 18, SITE_PHASE_DONE = 19,
                   SITE_ACT_READY = 20, SITE_TILE_READY = 21, SITE_TICKET = 22, SITE_FINISH = 23,
                   SITE_ABORTED = 24;

__device__ inline void fail(const PassArgs &a, unsigned *fl, int lane, unsigned site) {
  lds_st(&fl[F_ABORT], 1u, lane);
  if (lane == 0) {
    unsigned zero = 0;
    (void)__hip_atomic_compare_exchange_strong(&a.sync[SYNC_ERROR], &zero, site, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Wait until LDS word *p >= target; returns the value seen, or 0 after an
// abort or the 2 s bound (then the abort flags are set). target > 0.
__device__ inline unsigned wait_lds_ge(const PassArgs &a, unsigned *p, unsigned target, unsigned *fl, int lane,
                                       unsigned site) {
  unsigned v = lds_ld(p);
  if (v >= target) return v;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    v = lds_ld(p);
    if (v >= target) return v;
    if (lds_ld(&fl[F_ABORT])) {
      fail(a, fl, lane, SITE_ABORTED);
      return 0;
    }
    if (__builtin_amdgcn_s_memrealtime() - t0 > BARRIER_TIMEOUT_TICKS) {
      fail(a, fl, lane, site);
      return 0;
    }
  }
}

// The work-group's rectangle of a phase: row tiles [rt0, rt0 + rc) x k-tiles
// [k0, k0 + sc) of a projection of nrt x nkt tiles (rc = sc = 0: no work), its
// row group and k-group, and the k-groups of its row group that hold k-tiles.
struct Rect {
  int rt0, rc, k0, sc, rg, kg, nkg;
};

__device__ inline Rect cu_rect(const StreamShape &s, int nrt, int nkt, int x, int l, int per_xcd) {
  Rect r;
  r.rg = x * (per_xcd / s.gk) + l / s.gk;
  r.kg = l % s.gk;
  r.rt0 = r.rg * s.R;
  r.k0 = r.kg * s.S;
  r.rc = max(0, min(s.R, nrt - r.rt0));
  r.sc = max(0, min(s.S, nkt - r.k0));
  if (r.rc == 0 || r.sc == 0) r.rc = r.sc = 0;
  r.nkg = min(s.gk, (nkt + s.S - 1) / s.S);
  return r;
}

// ---------------------------------------------------------------------------
// Weight wave: tile t of the work-group's sequence (phases in order, each
// rectangle k-tile by k-tile, row tile by row tile) goes to slot t % NSLOT once
// the slot's previous tile has been consumed. Published (F_WPUB) when its
// loads have landed.
// ---------------------------------------------------------------------------
__device__ void produce_weights(const PassArgs &a, int np, uint8_t *ring, unsigned *fl, int x, int l, int lane) {
  uint32_t s = 0, pub = 0;
  for (int p = 0; p < np; ++p) {
    const int j = p & 3;
    const PhaseShape &ps = a.ph[j];
    const Rect r = cu_rect(a.ss[j], ps.nrt, ps.nkt, x, l, a.cus_per_xcd);
    if (r.rc == 0) continue;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.w[p >> 2][j], (short)0, ps.nrt * ps.nkt * TILE_BYTES, RAW_BUFFER_FLAGS);
    for (int jk = 0; jk < r.sc; ++jk) {
      for (int i = 0; i < r.rc; ++i) {
        const uint32_t q = s % NSLOT;
        if (s >= NSLOT) {
          const unsigned need = s / NSLOT;  // consumptions of slot q so far
          if (lds_ld(&fl[F_CONS + q]) < need) {
            // Publish everything that has landed before waiting for the slot.
            wait_vmcnt<0>();
            pub = s;
            lds_st(&fl[F_WPUB], pub, lane);
            if (!wait_lds_ge(a, &fl[F_CONS + q], need, fl, lane, SITE_WEIGHT_SLOT)) return;
          }
        }
        const uint32_t base = (uint32_t)(((r.rt0 + i) * ps.nkt + r.k0 + jk) * TILE_BYTES);
        uint8_t *t = ring + q * TILE_BYTES;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)t, 16, base + lane * 16, 0, 0, WEIGHT_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(t + CODE_HALF_BYTES), 16,
                                                 base + CODE_HALF_BYTES + lane * 16, 0, 0, WEIGHT_AUX);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(t + SCALE_OFFSET), 4,
                                                 base + SCALE_OFFSET + lane * 4, 0, 0, WEIGHT_AUX);
        ++s;
        if (s - pub > WLAG) {
          wait_vmcnt<3 * WLAG>();
          pub = s - WLAG;
          lds_st(&fl[F_WPUB], pub, lane);
        }
      }
    }
  }
  wait_vmcnt<0>();
  lds_st(&fl[F_WPUB], s, lane);
}

// ---------------------------------------------------------------------------
// Activation wave: before phase p > 0, waits for the work-group's consumers to
// finish phase p - 1 (their stores complete) and for the grid barrier; then
// loads the rectangle's k-tiles of packed activations into the activation ring
// (slot reuse waits for all four consumers), publishing each (F_APUB) when it
// has landed. After the last phase it counts the work-group finished; the last
// work-group to finish resets the barrier words and the XCD places.
// ---------------------------------------------------------------------------
template <int MB>
__device__ void produce_acts(const PassArgs &a, int np, uint8_t *aring, unsigned *fl, int x, int l, int lane) {
  constexpr int NA = n_act_slots<MB>(), ASB = act_slot_bytes<MB>(), LOADS = MB * 8;
  uint32_t s = 0, pub = 0;
  bool ok = true;
  for (int p = 0; p < np && ok; ++p) {
    const int j = p & 3;
    if (p > 0) {
      if (!wait_lds_ge(a, &fl[F_DONE], SC * p, fl, lane, SITE_PHASE_DONE)) return;
      unsigned pass = 1;
      if (lane == 0) {
        barrier_arrive(a.sync, (unsigned)p);
        pass = barrier_wait(a.sync, (unsigned)p) ? 1u : 0u;
      }
      if (!__builtin_amdgcn_readfirstlane(pass)) {
        lds_st(&fl[F_ABORT], 1u, lane);  // the barrier recorded its own site
        return;
      }
    }
    const PhaseShape &ps = a.ph[j];
    const Rect r = cu_rect(a.ss[j], ps.nrt, ps.nkt, x, l, a.cus_per_xcd);
    if (r.rc == 0) continue;
    const uint8_t *act = a.act0 + (size_t)(p >> 2) * a.layer_stride + a.act_off[j];
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, a.act_bytes[j], RAW_BUFFER_FLAGS);
    for (int jk = 0; jk < r.sc; ++jk) {
      const uint32_t q = s % NA;
      if (s >= NA) {
        const unsigned need = s - NA + 1;  // every consumer is done with k-tile s - NA
        unsigned least = lds_ld(&fl[F_APROG]);
        for (int w = 1; w < SC; ++w) least = min(least, lds_ld(&fl[F_APROG + w]));
        if (least < need) {
          wait_vmcnt<0>();
          pub = s;
          lds_st(&fl[F_APUB], pub, lane);
          for (int w = 0; w < SC; ++w)
            if (!wait_lds_ge(a, &fl[F_APROG + w], need, fl, lane, SITE_ACT_SLOT)) return;
        }
      }
      const uint32_t base = (uint32_t)((r.k0 + jk) * ASB);
      uint8_t *dst = aring + q * ASB;
#pragma unroll
      for (int c = 0; c < LOADS; ++c)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(dst + c * ACT_FRAG_BYTES), 16,
                                                 base + c * ACT_FRAG_BYTES + lane * 16, 0, 0, 0);
      ++s;
      if (s - pub > 1) {
        wait_vmcnt<LOADS>();
        pub = s - 1;
        lds_st(&fl[F_APUB], pub, lane);
      }
    }
    wait_vmcnt<0>();
    pub = s;
    lds_st(&fl[F_APUB], pub, lane);
  }
  // The consumers' last phase, then this work-group is finished.
  if (!wait_lds_ge(a, &fl[F_DONE], SC * np, fl, lane, SITE_FINISH)) return;
  if (lane == 0) {
    const unsigned done = __hip_atomic_fetch_add(&a.sync[SYNC_DONE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (done == gridDim.x - 1) {
      __hip_atomic_store(&a.sync[SYNC_RELEASE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.sync[SYNC_TOP], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      for (int gg = 0; gg < BARRIER_GROUPS; ++gg)
        __hip_atomic_store(&a.sync[SYNC_GROUP0 + 64 * gg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      for (int xx = 0; xx < 8; ++xx) {
        __hip_atomic_store(&a.counters[XCD_CNT + 16 * xx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        __hip_atomic_store(&a.counters[XCD_IDS + 16 * xx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      __hip_atomic_store(&a.sync[SYNC_DONE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

// ---------------------------------------------------------------------------
// Consumers.
// ---------------------------------------------------------------------------
// Bounded poll of a ticket word in the XCD's L2 until its low 16 bits reach
// `target`; false after an abort anywhere or the 2 s bound. The poll is an
// atomic add in the high 16 bits: an atomic executes in the L2 (a plain load
// could keep reading a stale L1 line), and one that changes the word cannot be
// turned into a load. Arrivals count in the low bits; the word is cleared with
// a store once every reader is done.
__device__ inline bool wait_ticket(const PassArgs &a, unsigned *cnt, unsigned target, unsigned *fl, int lane) {
  unsigned ok = 1;
  if (lane == 0) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((__hip_atomic_fetch_add(cnt, 0x10000u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) & 0xFFFFu) < target) {
      if (__hip_atomic_load(&a.sync[SYNC_ERROR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0 ||
          __builtin_amdgcn_s_memrealtime() - t0 > BARRIER_TIMEOUT_TICKS) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (__builtin_amdgcn_readfirstlane(ok)) return true;
  fail(a, fl, lane, SITE_TICKET);
  return false;
}

// Partial tile (row group rg, k-group kg, wave wv, slot) in the exchange buffer:
// MB 16x16 fp32 tiles in MFMA lane order (lane L's four values at 16 L bytes).
template <int MB>
__device__ inline int xoff(const StreamShape &s, int rg, int kg, int wv, int slot) {
  return ((((rg * s.gk + kg) * SC + wv) * SLOTS + slot) * MB) * 1024;
}

template <int MB>
__device__ inline void store_part(const PassArgs &a, int off, const f32x4 (&v)[MB], int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    *reinterpret_cast<f32x4 *>(reinterpret_cast<uint8_t *>(a.part) + off + mb * 1024 + lane * 16) = v[mb];
}

// Cache policy of the partial-tile loads: sc1 (agent scope). A persistent
// work-group reads the same partial lines again in later phases (the reducer
// role rotates), so the load must not be served by this CU's L1, which may
// still hold an earlier phase's values; agent scope goes past the L1 and is
// served by the XCD's L2, where the siblings' stores landed. (sc0 alone is
// workgroup scope, which the L1 of the work-group's own CU may serve.)
constexpr int PARTIAL_LOAD_AUX = 16;

template <int MB>
__device__ inline void load_part(__amdgpu_buffer_rsrc_t rp, int off, f32x4 (&v)[MB], int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(rp, off + mb * 1024 + lane * 16, 0, PARTIAL_LOAD_AUX);
    __builtin_memcpy(&v[mb], &x, 16);
  }
}

// Epilogue of one unit (row tile rt, or the (gate, up) pair rt, rt + 1).
template <int MB>
__device__ inline void unit_epilogue(const GemmArgs &g, int U, int rt, const f32x4 (&v0)[MB], const f32x4 (&v1)[MB],
                                     int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (U == 2)
      epi_pair_lane<MB>(v0[mb], v1[mb], rt, mb, lane, g.M, g.N, g.nrt, g.ts, g.C, g.epi);
    else
      epi_tile_lane<MB>(v0[mb], rt, mb, lane, g.M, g.N, g.nrt, g.ts, g.C, g.epi);
  }
}

template <int MB>
__device__ void consume(const PassArgs &a, int np, const uint8_t *ring, const uint8_t *aring, unsigned *fl, int w,
                        int x, int l, int lane) {
  constexpr int NA = n_act_slots<MB>(), ASB = act_slot_bytes<MB>();
  uint32_t tbase = 0, as = 0;
  unsigned wpub = 0, apub = 0;  // last published counts seen
  const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.part, (short)0, (int)(MAX_ROW_GROUPS * SC * SLOTS * MB * 1024), RAW_BUFFER_FLAGS);
  for (int p = 0; p < np; ++p) {
    const int j = p & 3;
    const PhaseShape &ps = a.ph[j];
    const StreamShape &ss = a.ss[j];
    const Rect r = cu_rect(ss, ps.nrt, ps.nkt, x, l, a.cus_per_xcd);
    if (r.rc > 0) {
      const int U = ss.unit;
      const int Uc = r.rc / U, q = Uc >> 2, e = Uc & 3;
      const int no = q * U, ne = e * U;  // own and leftover row slots
      f32x4 acc[SLOTS][MB];
#pragma unroll
      for (int i = 0; i < SLOTS; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[i][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

      for (int jk = 0; jk < r.sc; ++jk) {
        if (apub <= as) {
          apub = wait_lds_ge(a, &fl[F_APUB], as + 1, fl, lane, SITE_ACT_READY);
          if (!apub) return;
        }
        const uint4 *asl = reinterpret_cast<const uint4 *>(aring + (as % NA) * ASB);
        bf16x8 b[MB][8];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int qq = 0; qq < 8; ++qq) {
            const uint4 v = asl[(mb * 8 + qq) * 64 + lane];
            __builtin_memcpy(&b[mb][qq], &v, 16);
          }
        const uint32_t t0 = tbase + (uint32_t)(jk * r.rc);
        bool dead = false;
        // One weight tile (sequence number seq) into accumulator slot ac.
        auto tile = [&](uint32_t seq, f32x4 (&ac)[MB]) {
          if (wpub <= seq) {
            wpub = wait_lds_ge(a, &fl[F_WPUB], seq + 1, fl, lane, SITE_TILE_READY);
            if (!wpub) {
              dead = true;
              return;
            }
          }
          const uint8_t *t = ring + (seq % NSLOT) * TILE_BYTES;
          WTile wt;
          wt.c[0] = *reinterpret_cast<const uint4 *>(t + lane * 16);
          wt.c[1] = *reinterpret_cast<const uint4 *>(t + CODE_HALF_BYTES + lane * 16);
          wt.s = *reinterpret_cast<const uint32_t *>(t + SCALE_OFFSET + lane * 4);
          // LDS executes a wave's operations in order, so the slot is handed
          // back after these reads even though the count goes out before the
          // compute that uses them.
          lds_inc(&fl[F_CONS + seq % NSLOT], lane);
          compute_wtile<MB>(wt, b, ac);
        };
#pragma unroll
        for (int i = 0; i < OWN_SLOTS; ++i) {
          if (i < no && !dead) tile(t0 + (uint32_t)((w + 4 * (i / U)) * U + i % U), acc[i]);
        }
#pragma unroll
        for (int xi = 0; xi < EXTRA_SLOTS; ++xi) {
          const int xu = xi / U;
          if (xi < ne && !dead && (jk * e + xu) % SC == w)
            tile(t0 + (uint32_t)((4 * q + xu) * U + xi % U), acc[OWN_SLOTS + xi]);
        }
        if (dead) return;
        ++as;
        lds_st(&fl[F_APROG + w], as, lane);
      }
      tbase += (uint32_t)(r.rc * r.sc);

      // ---- reduction over k-groups (and, for leftover units, waves) ----
      const GemmArgs g = phase_gemm(a, p);
      const int kred = p % r.nkg;
      const bool reducer = r.kg == kred;
      unsigned *cnt = a.counters + RG_CNT + 8 * r.rg;
      if (!reducer) {
#pragma unroll
        for (int i = 0; i < OWN_SLOTS; ++i)
          if (i < no) store_part<MB>(a, xoff<MB>(ss, r.rg, r.kg, w, i), acc[i], lane);
      }
#pragma unroll
      for (int xi = 0; xi < EXTRA_SLOTS; ++xi)
        if (xi < ne) store_part<MB>(a, xoff<MB>(ss, r.rg, r.kg, w, OWN_SLOTS + xi), acc[OWN_SLOTS + xi], lane);
      const bool own_ticket = !reducer && no > 0;
      if (own_ticket || ne > 0) {
        // the partial stores are acknowledged by the L2 once the counter drains
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) {
          if (own_ticket) (void)__hip_atomic_fetch_add(cnt + w, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          if (ne > 0) (void)__hip_atomic_fetch_add(cnt + 4, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      if (reducer) {
        if (no > 0) {
          if (r.nkg > 1) {
            if (!wait_ticket(a, cnt + w, (unsigned)(r.nkg - 1), fl, lane)) return;
            if (lane == 0) __hip_atomic_store(cnt + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
            for (int i = 0; i < OWN_SLOTS; ++i) {
              if (i < no) {
                f32x4 v[MB];
                for (int kg2 = 0; kg2 < r.nkg; ++kg2) {
                  f32x4 y[MB];
                  if (kg2 == r.kg) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) y[mb] = acc[i][mb];
                  } else {
                    load_part<MB>(rp, xoff<MB>(ss, r.rg, kg2, w, i), y, lane);
                  }
#pragma unroll
                  for (int mb = 0; mb < MB; ++mb) v[mb] = kg2 == 0 ? y[mb] : v[mb] + y[mb];
                }
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[i][mb] = v[mb];
              }
            }
          }
#pragma unroll
          for (int i = 0; i < OWN_SLOTS; i += 2) {
            // slots i, i + 1: two row tiles, or one (gate, up) unit when U = 2
            if (i < no) {
              const int rt = r.rt0 + (w + 4 * (i / U)) * U + i % U;
              if (U == 2) {
                unit_epilogue<MB>(g, 2, rt, acc[i], acc[i + 1], lane);
              } else {
                unit_epilogue<MB>(g, 1, rt, acc[i], acc[i], lane);
                if (i + 1 < no) unit_epilogue<MB>(g, 1, r.rt0 + w + 4 * (i + 1), acc[i + 1], acc[i + 1], lane);
              }
            }
          }
        }
        if (ne > 0 && w < e) {
          // leftover unit w: every wave of every k-group published a partial
          if (!wait_ticket(a, cnt + 4, (unsigned)(SC * r.nkg), fl, lane)) return;
          f32x4 v[2][MB];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            if (t < U) {
              bool first = true;
              for (int kg2 = 0; kg2 < r.nkg; ++kg2)
                for (int w2 = 0; w2 < SC; ++w2) {
                  f32x4 y[MB];
                  load_part<MB>(rp, xoff<MB>(ss, r.rg, kg2, w2, OWN_SLOTS + w * U + t), y, lane);
#pragma unroll
                  for (int mb = 0; mb < MB; ++mb) v[t][mb] = first ? y[mb] : v[t][mb] + y[mb];
                  first = false;
                }
            }
          }
          const int rt = r.rt0 + (4 * q + w) * U;
          if (U == 2) {
            unit_epilogue<MB>(g, 2, rt, v[0], v[1], lane);
          } else {
            unit_epilogue<MB>(g, 1, rt, v[0], v[0], lane);
          }
          // The last of the e readers clears both words for the next phase
          // (every reader has finished polling by then).
          if (lane == 0) {
            const unsigned old = __hip_atomic_fetch_add(cnt + 5, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (old == (unsigned)(e - 1)) {
              __hip_atomic_store(cnt + 4, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              __hip_atomic_store(cnt + 5, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        }
      }
    }
    // This wave's stores of the phase are complete before its arrival.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_inc(&fl[F_DONE], lane);
  }
}

template <int MB>
__global__ __launch_bounds__(SW_THREADS) void k_stream(PassArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t *ring = lds;
  uint8_t *aring = lds + NSLOT * TILE_BYTES;
  unsigned *fl = reinterpret_cast<unsigned *>(aring + n_act_slots<MB>() * act_slot_bytes<MB>());
  __shared__ unsigned place;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int np = 4 * a.n_layers;
  for (int i = tid; i < F_WORDS; i += SW_THREADS) fl[i] = 0u;
  if (tid == 0) {
    // A place on the XCD this work-group runs on: the gk work-groups of a row
    // group are places of one XCD, whatever order the work-groups were dealt
    // in. The hardware's XCD ids need not be 0..7, so the first work-group
    // of each XCD claims the next free index x in a table of ids.
    const unsigned hw = ((unsigned)__builtin_amdgcn_s_getreg(XCC_ID_HWREG) & 0xFFFFu) + 1u;
    unsigned xx = 8;
    for (unsigned i = 0; i < 8u; ++i) {
      unsigned seen = 0;
      (void)__hip_atomic_compare_exchange_strong(&a.counters[XCD_IDS + 16 * i], &seen, hw, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      if (seen == 0 || seen == hw) {
        xx = i;
        break;
      }
    }
    unsigned ll = 0xFFFFu;
    if (xx < 8u)
      ll = __hip_atomic_fetch_add(&a.counters[XCD_CNT + 16 * xx], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    place = (xx << 16) | (ll & 0xFFFFu);
  }
  __syncthreads();
  const int x = __builtin_amdgcn_readfirstlane((int)(place >> 16));
  const int l = __builtin_amdgcn_readfirstlane((int)(place & 0xFFFFu));
  if (x >= 8 || l >= a.cus_per_xcd) {
    // More than 8 XCDs, or more work-groups on one XCD than it has CUs: the
    // places cannot be assigned; report it (nvfp4v_pass_status) and leave.
    if (tid == 0) {
      unsigned zero = 0;
      (void)__hip_atomic_compare_exchange_strong(&a.sync[SYNC_ERROR], &zero, SITE_PLACE, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  if (wave == SC) {
    produce_weights(a, np, ring, fl, x, l, lane);
    wait_vmcnt<0>();
  } else if (wave == SC + 1) {
    produce_acts<MB>(a, np, aring, fl, x, l, lane);
    wait_vmcnt<0>();
  } else {
    consume<MB>(a, np, ring, aring, fl, wave, x, l, lane);
  }
}

__global__ void k_zero_words(unsigned *w, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

typedef void (*StreamKernel)(PassArgs);

// The rectangle of a projection of nrt x nkt tiles for G = 8 * per_xcd
// work-groups: the k-group count gk (a divisor of per_xcd) that gives the
// busiest work-group the fewest tiles (ties: fewer k-groups), with a consumer
// wave's own rows and the leftover rows within the accumulator slots in every
// row group (including a short last one). False if no gk fits.
bool choose_stream_shape(int64_t nrt, int64_t nkt, int unit, int per_xcd, StreamShape *out) {
  const int G = 8 * per_xcd;
  int64_t best = INT64_MAX;
  for (int gk = 1; gk <= 8; gk *= 2) {
    if (per_xcd % gk) continue;
    const int nrg = G / gk;
    if (nrg > MAX_ROW_GROUPS) continue;
    int64_t R = (nrt + nrg - 1) / nrg;
    R = (R + unit - 1) / unit * unit;
    const int64_t S = (nkt + gk - 1) / gk;
    auto fits = [&](int64_t rc) {
      const int64_t uc = rc / unit;
      return (uc / 4) * unit <= OWN_SLOTS && (uc % 4) * unit <= EXTRA_SLOTS;
    };
    const int64_t used = (nrt + R - 1) / R;
    if (!fits(R) || !fits(nrt - (used - 1) * R)) continue;
    const int64_t cost = R * S;
    if (cost < best) {
      best = cost;
      *out = StreamShape{gk, (int)R, (int)S, unit};
    }
  }
  return best != INT64_MAX;
}

}  // namespace

namespace nvfp4v {
namespace passk {

int stream_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t H, int64_t I,
                const uint16_t *h0, int64_t m, const PassWs &w, uint16_t *h_out, uint16_t *trace,
                hipStream_t stream) {
  const int mb = (int)((m + 15) / 16);
  StreamKernel kern = mb == 1 ? k_stream<1> : mb == 2 ? k_stream<2> : nullptr;
  if (!kern) return NVFP4V_E_M_RANGE;
  const size_t lds = mb == 1 ? stream_lds_bytes<1>() : stream_lds_bytes<2>();
  if (ctx->num_cus % 8 || ctx->num_cus / 8 < 1) return NVFP4V_E_HIP;
  const int per_xcd = ctx->num_cus / 8;
  const int grid = ctx->num_cus;
  hipError_t e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return hip_status(ctx, e);
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kern, SW_THREADS, lds);
  if (e != hipSuccess) return hip_status(ctx, e);
  if (per_cu < 1) return NVFP4V_E_HIP;
  Layout ls[4];
  if (!make_layout(3 * H, H, &ls[0]) || !make_layout(H, H, &ls[1]) || !make_layout(2 * I, H, &ls[2]) ||
      !make_layout(H, I, &ls[3]))
    return NVFP4V_E_SHAPE;
  PassArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = (int)m;
  a.H = (int)H;
  a.last_layer = n_layers - 1;
  a.cus_per_xcd = per_xcd;
  for (int j = 0; j < 4; ++j) {
    if (ls[j].bytes() > (size_t)0x7FFF0000) return NVFP4V_E_SHAPE;  // 32-bit buffer offsets
    a.ph[j].N = (int)ls[j].n;
    a.ph[j].nrt = (int)ls[j].nrt;
    a.ph[j].nkt = (int)ls[j].nkt;
    if (!choose_stream_shape(ls[j].nrt, ls[j].nkt, j == 2 ? 2 : 1, per_xcd, &a.ss[j])) return NVFP4V_E_SHAPE;
    if (w.act_bytes[j] > (size_t)0x7FFF0000) return NVFP4V_E_SHAPE;
  }
  const size_t part_need = (size_t)MAX_ROW_GROUPS * SC * SLOTS * mb * 256;
  if (part_need > ctx->partial_floats || (size_t)STREAM_COUNTER_WORDS > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  a.cst[0] = a.cst[1] = (float)(1.0 / std::sqrt((double)H));
  a.cst[2] = (float)(1.0 / std::sqrt(2.0 * (double)H));
  a.cst[3] = (float)(1.0 / std::sqrt((double)I));
  a.layer_stride = w.layer_stride;
  for (int j = 0; j < 4; ++j) {
    a.act_off[j] = w.act_off[j];
    a.act_bytes[j] = (int)w.act_bytes[j];
    a.C[j] = w.C[j];
  }
  a.h_out = h_out;
  a.trace = trace;
  a.trace_m = (int)w.trace_m;
  a.part = ctx->partials;
  a.counters = ctx->counters;
  a.sync = ctx->pass_sync;
  a.timeline = nullptr;
  ctx->last_pass_grid = grid;
  ctx->last_pass_phases = 4 * n_layers;
  if (fault_injected()) return NVFP4V_E_FAULT;

  // The barrier words (zeroed by the packing kernel) and this mode's counters
  // start every pass at zero, also after a pass that gave up.
  hipLaunchKernelGGL(k_zero_words, dim3(8), dim3(256), 0, stream, ctx->counters, STREAM_COUNTER_WORDS);
  int rc = hip_status(ctx, hipGetLastError());
  if (!rc) rc = launch_pack_act(ctx, h0, m, H, w.act0, stream, ctx->pass_sync);
  for (int l0 = 0; l0 < n_layers && rc == NVFP4V_OK; l0 += LAYERS_PER_LAUNCH) {
    a.layer0 = l0;
    a.n_layers = std::min(LAYERS_PER_LAUNCH, n_layers - l0);
    for (int l = 0; l < a.n_layers; ++l) {
      const nvfp4v_layer &L = layers[l0 + l];
      a.w[l][0] = (const uint8_t *)L.qkv;
      a.w[l][1] = (const uint8_t *)L.o;
      a.w[l][2] = (const uint8_t *)L.gate_up;
      a.w[l][3] = (const uint8_t *)L.down;
      a.ts[l][0] = L.ts_qkv;
      a.ts[l][1] = L.ts_o;
      a.ts[l][2] = L.ts_gate_up;
      a.ts[l][3] = L.ts_down;
    }
    a.act0 = w.act0 + (size_t)l0 * w.layer_stride;
    a.phase0 = 4 * l0;
    void *args[] = {&a};
    e = hipLaunchCooperativeKernel((const void *)kern, dim3((unsigned)grid), dim3(SW_THREADS), args, (unsigned)lds,
                                   stream);
    rc = hip_status(ctx, e);
  }
  return rc;
}

}  // namespace passk
}  // namespace nvfp4v
