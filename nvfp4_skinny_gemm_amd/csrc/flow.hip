// The verify pass in flow mode: one persistent, cooperatively launched kernel
// per 32 layers in which the weight stream never waits for a phase boundary.
//
// The pass reads 0.5625 bytes per weight and almost nothing else, so its
// speed is set by how steadily HBM is kept busy (TandemLLM manual, "What
// TandemLLM is", 1.2 "Two levers": 16 draft rows cost about what one does).
// Its 4 GEMMs per layer depend on each other only through their activations,
// never through the weights. A work-group therefore splits into roles:
//
//  * one producer wave streams the work-group's weight tiles, in the order the
//    work-group will use them across all phases of the launch, from HBM
//    straight into a ring of LDS slots with buffer_load ... lds (no VGPRs),
//    keeping two slots of loads in flight. It waits only for a free slot; it
//    never waits for another work-group, so while the consumers sit at a phase
//    boundary the next phase's weights keep arriving.
//  * WC consumer waves each own R row tiles of the slot's RT = WC R row tiles
//    (waves split N): per k-tile a consumer reads its tiles from the slot,
//    loads the k-tile's activation fragments (from L2, shared with the other
//    consumers through the CU's L1), dequantises in registers and runs the
//    MFMAs exactly as the per-call GEMM does.
//
// Work split: every phase's (row block x k-tile) units, in row-block-major
// order, are cut into one equal contiguous range per work-group (a stream-K
// schedule), so every work-group streams the same bytes per phase. A row block
// spread over several work-groups is summed from their partial tiles in k
// order by the last one to arrive (per consumer wave, with a system-scope
// ticket), so the result is bitwise reproducible. A work-group crosses to
// phase p + 1 once every work-group has finished phase p: each consumer wave
// counts its arrival in LDS, the last one arrives at the grid barrier (the
// same hierarchical barrier as the other persistent kernel) and publishes the
// release in LDS.
//
// Coherence without fences is as in the other persistent kernel: epilogues
// and partial sums are written with system-coherent stores, every phase reads
// activations from a buffer of its own, partials are read with system-coherent
// loads, and every wait is bounded (2 s), after which an error flag is set and
// every wave leaves.
#include <hip/hip_bf16.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>

#include "pass_common.h"

using namespace nvfp4v;
using namespace nvfp4v::dev;
using namespace nvfp4v::passk;

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// LDS words after the ring: per slot a count of consumer reads (consumers add
// 1 each time they are done with it) and the generation the producer last
// filled it for; then the work-group's arrival count, the released phase and
// its finish count.
template <int NSLOT>
struct FlowFlags {
  static constexpr int CONSUMED = 0, FULL = NSLOT, ARRIVE = 2 * NSLOT, READY = 2 * NSLOT + 1,
                       FINISH = 2 * NSLOT + 2, WORDS = 2 * NSLOT + 4;
};
constexpr unsigned READY_ABORT = 0xFFFFFFFFu;

// LDS flag accesses are written out so that the compiler's wait-count pass
// does not treat them as reads of the LDS the producer's loads are filling
// (it would wait for every load in flight before each one).
__device__ inline uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }
__device__ inline unsigned lds_load(const unsigned *p) {
  unsigned v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ inline void lds_store(unsigned *p, unsigned v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_addr(p)), "v"(v) : "memory");
}
// Adds v once for the wave (lane 0) and returns the previous value to every lane.
__device__ inline unsigned lds_add_wave(unsigned *p, unsigned v, int lane) {
  unsigned old = 0;
  if (lane == 0)
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(old) : "v"(lds_addr(p)), "v"(v) : "memory");
  return __builtin_amdgcn_readfirstlane(old);
}

__device__ inline bool timed_out(uint64_t t0) {
  return __builtin_amdgcn_s_memrealtime() - t0 > BARRIER_TIMEOUT_TICKS;
}

__device__ inline void set_error(unsigned *sync) {
  __hip_atomic_store(&sync[SYNC_ERROR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// s_waitcnt with vmcnt = N (lgkmcnt and expcnt left open).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The range of units of work-group b in one phase and the work-group that
// holds unit x (ranges are [T b / G, T (b + 1) / G)).
__device__ inline int64_t uni64(int64_t x);
__device__ inline int uni(int x);
__device__ inline void flow_range(const FlowShape &f, int b, int G, int64_t *lo, int64_t *hi) {
  *lo = uni64(f.T * b / G);
  *hi = uni64(f.T * (b + 1) / G);
}
__device__ inline int flow_owner(const FlowShape &f, int64_t x, int G) { return uni((int)(((x + 1) * G - 1) / f.T)); }

// Position in a work-group's sequence of items (one k-tile of one row block
// of one phase); p == np past the end.
struct FlowIt {
  int p;
  int64_t pos, hi;  // current piece starts at unit pos; the phase's range ends at hi
  int rb, kA, kB, kt;
};

// Wave-uniform copies (the 64-bit divisions run on the vector ALU; keeping
// the results in scalar registers keeps every address derived from them, and
// the kernel-argument loads indexed by the phase, scalar).
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ inline void flow_piece(FlowIt &it, const FlowShape &f) {
  it.rb = uni((int)(it.pos / f.nkt));
  it.kA = uni((int)(it.pos - (int64_t)it.rb * f.nkt));
  it.kB = uni((int)std::min<int64_t>(f.nkt, it.kA + (it.hi - it.pos)));
  it.kt = it.kA;
}

// First item of phase p or later.
__device__ inline void flow_seek(FlowIt &it, const PassArgs &a, int p, int np, int b, int G) {
  for (; p < np; ++p) {
    int64_t lo, hi;
    flow_range(a.fs[p & 3], b, G, &lo, &hi);
    if (lo < hi) {
      it.p = p, it.pos = lo, it.hi = hi;
      flow_piece(it, a.fs[p & 3]);
      return;
    }
  }
  it.p = np;
}

__device__ inline void flow_next(FlowIt &it, const PassArgs &a, int np, int b, int G) {
  if (++it.kt < it.kB) return;
  it.pos += it.kB - it.kA;
  if (it.pos < it.hi) {
    flow_piece(it, a.fs[it.p & 3]);
    return;
  }
  flow_seek(it, a, it.p + 1, np, b, G);
}

// ---------------------------------------------------------------------------
// Producer: fill slot s % NSLOT with the RT weight tiles of item s, in item
// order, once the consumers are done with the slot's previous item; mark slot
// s full when its loads have landed (LAG slots of loads stay in flight).
// ---------------------------------------------------------------------------
template <int WC, int RT, int NSLOT, int LAG>
__device__ __attribute__((always_inline)) inline void flow_produce(const PassArgs &a, int np, uint8_t *ring, unsigned *fl, int lane) {
  using F = FlowFlags<NSLOT>;
  constexpr int SLOT = RT * TILE_BYTES;
  constexpr int LOADS = 3 * RT;  // per slot: two 1 KiB code halves and 256 bytes of scales per tile
  static_assert(LOADS * LAG < 64, "loads in flight exceed the vmcnt range");
  const int b = blockIdx.x, G = gridDim.x;
  uint32_t s = 0;
  FlowIt it;
  flow_seek(it, a, 0, np, b, G);
  while (it.p < np) {
    const FlowShape &f = a.fs[it.p & 3];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.w[it.p >> 2][it.p & 3], (short)0, f.nrt * f.nkt * TILE_BYTES, RAW_BUFFER_FLAGS);
    const int q = (int)(s % NSLOT);
    const uint32_t u = s / NSLOT;
    if (u > 0) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (lds_load(&fl[F::CONSUMED + q]) < WC * u) {
        if (lds_load(&fl[F::READY]) == READY_ABORT || timed_out(t0)) {
          set_error(a.sync);
          wait_vmcnt<0>();
          return;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    uint8_t *dst = ring + q * SLOT;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int rt = it.rb * RT + i;
      const uint32_t base = rt < f.nrt ? (uint32_t)(rt * f.nkt + it.kt) * TILE_BYTES : (uint32_t)OOB;
      uint8_t *t = dst + i * TILE_BYTES;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)t, 16, base + lane * 16, 0, 0, WEIGHT_AUX);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(t + CODE_HALF_BYTES), 16,
                                               base + CODE_HALF_BYTES + lane * 16, 0, 0, WEIGHT_AUX);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(t + SCALE_OFFSET), 4,
                                               base + SCALE_OFFSET + lane * 4, 0, 0, WEIGHT_AUX);
    }
    ++s;
    if (s > LAG) {
      wait_vmcnt<LOADS * LAG>();
      const uint32_t d = s - 1 - LAG;
      lds_store(&fl[F::FULL + d % NSLOT], d / NSLOT + 1);
    }
    flow_next(it, a, np, b, G);
  }
  wait_vmcnt<0>();
  for (uint32_t d = s > LAG ? s - LAG : 0; d < s; ++d) lds_store(&fl[F::FULL + d % NSLOT], d / NSLOT + 1);
}

// ---------------------------------------------------------------------------
// Consumers.
// ---------------------------------------------------------------------------
template <int R>
__device__ __attribute__((always_inline)) inline void read_slot(WTile (&w)[R], const uint8_t *slot, int tile0, int lane) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint8_t *t = slot + (tile0 + r) * TILE_BYTES;
    w[r].c[0] = *reinterpret_cast<const uint4 *>(t + lane * 16);
    w[r].c[1] = *reinterpret_cast<const uint4 *>(t + CODE_HALF_BYTES + lane * 16);
    w[r].s = *reinterpret_cast<const uint32_t *>(t + SCALE_OFFSET + lane * 4);
  }
}

__device__ inline __amdgpu_buffer_rsrc_t act_rsrc(const PassArgs &a, int p) {
  const int j = p & 3;
  const uint8_t *act = a.act0 + (size_t)(p >> 2) * a.layer_stride + a.act_off[j];
  return __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, a.act_bytes[j], RAW_BUFFER_FLAGS);
}

// One k-tile of this wave's R row tiles (weights w, activation fragments b of
// the k-tile), MFMA by MFMA: fragment q of every 16-row block serves all R
// tiles, and right after its last use it is refilled with fragment q of
// k-tile kt_next (zeros when `refill` is false), so the refill has a whole
// k-tile of compute to arrive in and only one copy of the fragments is live.
// Each accumulator takes its MFMAs in the same order as compute_wtile.
template <int MB, int R>
__device__ __attribute__((always_inline)) inline void compute_roll(const WTile (&w)[R], bf16x8 (&b)[MB][8],
                                                                   f32x4 (&acc)[R][MB],
                                                                   __amdgpu_buffer_rsrc_t ra, int kt_next,
                                                                   bool refill, int M, int lane) {
  float sc[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r) scales4(w[r].s, sc[r]);
  const int col = lane & 15;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q = 4 * c + j;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t cw = c == 0 ? (j == 0 ? w[r].c[0].x : j == 1 ? w[r].c[0].y : j == 2 ? w[r].c[0].z : w[r].c[0].w)
                                   : (j == 0 ? w[r].c[1].x : j == 1 ? w[r].c[1].y : j == 2 ? w[r].c[1].z : w[r].c[1].w);
        const bf16x8 wf = dequant8(cw, sc[r][2 * c + (j >> 1)]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, b[mb][q], acc[r][mb], 0, 0, 0);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bool v = refill && mb * 16 + col < M;
        const int off = v ? ((kt_next * MB + mb) * 8 + q) * ACT_FRAG_BYTES + lane * 16 : OOB;
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
        __builtin_memcpy(&b[mb][q], &x, 16);
      }
    }
}

// Final values of this wave's R row tiles (row tiles rt0 .. rt0 + R - 1).
template <int MB, int R>
__device__ __attribute__((always_inline)) inline void flow_epilogue(const f32x4 (&v)[R][MB], const GemmArgs &g, int rt0, int lane) {
  if (g.epi.mode == EPI_PAIR) {
#pragma unroll
    for (int r = 0; r < R; r += 2)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        epi_pair_lane<MB>(v[r][mb], v[r + 1][mb], rt0 + r, mb, lane, g.M, g.N, g.nrt, g.ts, g.C, g.epi);
    return;
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) epi_tile_lane<MB>(v[r][mb], rt0 + r, mb, lane, g.M, g.N, g.nrt, g.ts, g.C, g.epi);
}

// End of this wave's part of a piece (row block it.rb, k-tiles [kA, kB) of
// phase it.p). A row block held by one work-group ends here; otherwise the
// wave publishes its partial tiles, takes a ticket, and the last of the row
// block's pieces to arrive sums them in piece (k) order. Leaves acc zeroed.
template <int MB, int WC, int R>
__device__ __attribute__((always_inline)) inline void flow_flush(const PassArgs &a, const FlowIt &it, f32x4 (&acc)[R][MB], int w, int lane) {
  constexpr int RT = WC * R;
  const FlowShape &f = a.fs[it.p & 3];
  const int G = gridDim.x, b = blockIdx.x;
  const GemmArgs g = phase_gemm(a, it.p);
  const int rt0 = it.rb * RT + w * R;
  // The row block's pieces and this one's index among them (k order). With
  // at least one unit per work-group (T >= G) every work-group between the
  // owners of the row block's first and last units holds one piece; with
  // fewer units than work-groups every unit is a piece of its own.
  int nq, jq;
  if (f.T >= G) {
    const int64_t first = (int64_t)it.rb * f.nkt;
    const int b0 = flow_owner(f, first, G), b1 = flow_owner(f, first + f.nkt - 1, G);
    nq = b1 - b0 + 1, jq = b - b0;
  } else {
    nq = f.nkt, jq = it.kA;
  }
  if (nq == 1) {
    flow_epilogue<MB, R>(acc, g, rt0, lane);
  } else {
    constexpr int FLOATS = R * MB * 256;  // this wave's partial tiles
    float *mine = a.part + ((size_t)(it.rb * f.nq_max + jq) * WC + w) * FLOATS;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float *dst = mine + ((r * MB + mb) * 64 + lane) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) __hip_atomic_store(dst + e, acc[r][mb][e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    // The partial stores have reached memory once this wave's counters drain.
    __builtin_amdgcn_s_waitcnt(0);
    unsigned *ticket = &a.counters[it.rb * WC + w];
    unsigned t = 0;
    if (lane == 0) t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t == (unsigned)(nq - 1)) {
      f32x4 v[R][MB];
      const float *row0 = a.part + ((size_t)(it.rb * f.nq_max) * WC + w) * FLOATS;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const float *src = row0 + ((r * MB + mb) * 64 + lane) * 4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[r][mb][e] = __hip_atomic_load(src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          for (int j = 1; j < nq; ++j) {
            const float *sj = src + (size_t)j * WC * FLOATS;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[r][mb][e] += __hip_atomic_load(sj + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          }
        }
      if (lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      flow_epilogue<MB, R>(v, g, rt0, lane);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Arrive for every phase before `target` not yet arrived for, waiting for
// each to be released (the work-group's last consumer wave to arrive takes
// the grid barrier and publishes the release). False after an abort.
template <int WC, int NSLOT>
__device__ __attribute__((always_inline)) inline bool flow_sync_to(const PassArgs &a, int target, int &synced, unsigned *fl, int lane) {
  using F = FlowFlags<NSLOT>;
  while (synced < target) {
    const unsigned q = (unsigned)synced;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores of phase q have completed
    const unsigned old = lds_add_wave(&fl[F::ARRIVE], 1u, lane);
    if (old + 1 == WC * (q + 1)) {
      unsigned rel = 0;
      if (lane == 0) {
        if (a.timeline && blockIdx.x < PASS_TIMELINE_WGS && a.phase0 + q < PASS_TIMELINE_PHASES)
          a.timeline[((size_t)(a.phase0 + q) * PASS_TIMELINE_WGS + blockIdx.x) * 2 + 1] = __builtin_amdgcn_s_memrealtime();
        barrier_arrive(a.sync, q + 1);
        rel = barrier_wait(a.sync, q + 1) ? q + 1 : READY_ABORT;
        if (a.timeline && blockIdx.x < PASS_TIMELINE_WGS && a.phase0 + q + 1 < PASS_TIMELINE_PHASES)
          a.timeline[((size_t)(a.phase0 + q + 1) * PASS_TIMELINE_WGS + blockIdx.x) * 2] = __builtin_amdgcn_s_memrealtime();
      }
      rel = __builtin_amdgcn_readfirstlane(rel);
      if (lane == 0) lds_store(&fl[F::READY], rel);
      if (rel == READY_ABORT) return false;
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        const unsigned r = lds_load(&fl[F::READY]);
        if (r == READY_ABORT) return false;
        if (r >= q + 1) break;
        if (timed_out(t0)) {
          set_error(a.sync);
          if (lane == 0) lds_store(&fl[F::READY], READY_ABORT);
          return false;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    ++synced;
  }
  return true;
}

// Wait until the producer has filled slot s (generation s / NSLOT + 1).
template <int NSLOT>
__device__ __attribute__((always_inline)) inline bool flow_wait_full(const PassArgs &a, unsigned *fl, uint32_t s, int lane) {
  using F = FlowFlags<NSLOT>;
  const unsigned gen = s / NSLOT + 1;
  if (lds_load(&fl[F::FULL + s % NSLOT]) >= gen) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_load(&fl[F::FULL + s % NSLOT]) >= gen) return true;
    if (lds_load(&fl[F::READY]) == READY_ABORT) return false;
    if (timed_out(t0)) {
      set_error(a.sync);
      if (lane == 0) lds_store(&fl[F::READY], READY_ABORT);
      return false;
    }
  }
}

// First phase at or after p in which work-group b has work (np if none).
__device__ inline int flow_next_phase(const PassArgs &a, int p, int np, int b, int G) {
  for (; p < np; ++p) {
    int64_t lo, hi;
    flow_range(a.fs[p & 3], b, G, &lo, &hi);
    if (lo < hi) return p;
  }
  return np;
}

template <int MB, int WC, int R, int NSLOT>
__device__ __attribute__((always_inline)) inline void flow_consume(const PassArgs &a, int np, const uint8_t *ring,
                                                                   unsigned *fl, int w, int lane) {
  using F = FlowFlags<NSLOT>;
  constexpr int RT = WC * R;
  constexpr int SLOT = RT * TILE_BYTES;
  const int b = blockIdx.x, G = gridDim.x;
  const int M = a.M;
  int synced = 0;  // phases < synced have been released
  int p = flow_next_phase(a, 0, np, b, G);
  if (p < np) {
    f32x4 acc[R][MB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    WTile w0[R], w1[R];
    bf16x8 act[MB][8];
    uint32_t s = 0;  // slot sequence number of the current item
    if (!flow_wait_full<NSLOT>(a, fl, 0, lane)) return;
    read_slot<R>(w0, ring, w * R, lane);
    while (p < np) {
      const int pn = flow_next_phase(a, p + 1, np, b, G);  // the phase after this one
      if (!flow_sync_to<WC, NSLOT>(a, p, synced, fl, lane)) return;
      const FlowShape &f = a.fs[p & 3];
      const int nkt = f.nkt;
      int64_t lo, hi;
      flow_range(f, b, G, &lo, &hi);
      const __amdgpu_buffer_rsrc_t ra = act_rsrc(a, p);
      load_afrag<MB>(act, ra, (int)(lo % nkt), true, M, lane);
      for (int64_t pos = lo; pos < hi;) {
        FlowIt it;
        it.p = p, it.pos = pos, it.hi = hi;
        flow_piece(it, f);
        const int kA = it.kA, kB = it.kB;
        const bool last_piece = pos + (kB - kA) >= hi;
        const bool more = !last_piece || pn < np;  // an item follows this piece
        // One item (k-tile kt): request the next item's weights from its slot,
        // compute this one while refilling the fragments with the next item's
        // when it is in this phase, then hand the slot back.
#define NVFP4V_FLOW_STEP(WCUR, WNXT)                                                                 \
  {                                                                                                   \
    const bool in_piece = kt + 1 < kB;                                                                \
    if (in_piece || more) {                                                                           \
      if (!flow_wait_full<NSLOT>(a, fl, s + 1, lane)) return;                                         \
    }                                                                                                 \
    /* read on every path (unused past the last item) so the wait counts stay exact */               \
    read_slot<R>(WNXT, ring + ((s + 1) % NSLOT) * SLOT, w * R, lane);                                 \
    __builtin_amdgcn_sched_barrier(0); /* keep the reads ahead of this item's compute */            \
    compute_roll<MB, R>(WCUR, act, acc, ra, in_piece ? kt + 1 : 0, in_piece || !last_piece, M, lane); \
    if (lane == 0) {                                                                                  \
      asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(&fl[F::CONSUMED + s % NSLOT])), "v"(1u)         \
                   : "memory");                                                                       \
    }                                                                                                 \
    ++s;                                                                                              \
    ++kt;                                                                                             \
  }
        int kt = kA;
        for (;;) {
          NVFP4V_FLOW_STEP(w0, w1)
          if (kt >= kB) {
#pragma unroll
            for (int r = 0; r < R; ++r) w0[r] = w1[r];  // the next item's weights back in w0
            break;
          }
          NVFP4V_FLOW_STEP(w1, w0)
          if (kt >= kB) break;
        }
#undef NVFP4V_FLOW_STEP
        flow_flush<MB, WC, R>(a, it, acc, w, lane);
        pos += kB - kA;
      }
      p = pn;
    }
  }
  flow_sync_to<WC, NSLOT>(a, np - 1, synced, fl, lane);
}

template <int MB, int WC, int R, int NSLOT, int LAG>
__global__ __launch_bounds__((WC + 1) * 64) void k_flow(PassArgs a) {
  using F = FlowFlags<NSLOT>;
  constexpr int RT = WC * R;
  extern __shared__ __align__(16) uint8_t lds[];
  uint8_t *ring = lds;
  unsigned *fl = reinterpret_cast<unsigned *>(lds + NSLOT * RT * TILE_BYTES);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int np = 4 * a.n_layers;
  for (int i = tid; i < F::WORDS; i += (WC + 1) * 64) fl[i] = 0u;
  if (a.timeline && tid == 0 && blockIdx.x < PASS_TIMELINE_WGS && a.phase0 < (int)PASS_TIMELINE_PHASES)
    a.timeline[((size_t)a.phase0 * PASS_TIMELINE_WGS + blockIdx.x) * 2] = __builtin_amdgcn_s_memrealtime();
  __syncthreads();
  if (wave == WC) {
    flow_produce<WC, RT, NSLOT, LAG>(a, np, ring, fl, lane);
    return;
  }
  flow_consume<MB, WC, R, NSLOT>(a, np, ring, fl, wave, lane);
  // The last consumer wave of the last work-group to finish resets the barrier
  // words for the next launch (every work-group has passed every barrier).
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned old = lds_add_wave(&fl[F::FINISH], 1u, lane);
  if (old + 1 == WC && lane == 0) {
    const unsigned done =
        __hip_atomic_fetch_add(&a.sync[SYNC_DONE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (done == gridDim.x - 1) {
      __hip_atomic_store(&a.sync[SYNC_RELEASE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.sync[SYNC_TOP], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      for (int gg = 0; gg < BARRIER_GROUPS; ++gg)
        __hip_atomic_store(&a.sync[SYNC_GROUP0 + 64 * gg], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(&a.sync[SYNC_DONE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

typedef void (*FlowKernel)(PassArgs);

struct FlowConfig {
  FlowKernel kern;
  int wc, r, nslot;
};

// Consumer waves x row tiles per wave: 4 x 2 (8 row tiles, 18 KiB per slot,
// an 8-slot ring of 144 KiB).
bool pick_flow(int mb, FlowConfig *c) {
  c->wc = 4, c->r = 2, c->nslot = 8;
  switch (mb) {
    case 1: c->kern = k_flow<1, 4, 2, 8, 2>; return true;
    case 2: c->kern = k_flow<2, 4, 2, 8, 2>; return true;
    default: return false;
  }
}

size_t flow_lds_bytes(const FlowConfig &c) {
  return (size_t)c.nslot * c.wc * c.r * TILE_BYTES + 4 * (2 * c.nslot + 4);
}

FlowShape flow_shape(int64_t nrt, int64_t nkt, int rt_per_block, int G) {
  FlowShape f;
  f.nrt = (int)nrt;
  f.nkt = (int)nkt;
  f.nrb = (int)((nrt + rt_per_block - 1) / rt_per_block);
  f.T = (int64_t)f.nrb * nkt;
  f.nq_max = 1;
  if (f.T < G) {  // every unit is a piece of its own
    f.nq_max = f.nkt;
    return f;
  }
  for (int rb = 0; rb < f.nrb; ++rb) {
    const int64_t first = (int64_t)rb * nkt, last = first + nkt - 1;
    const int64_t b0 = ((first + 1) * G - 1) / f.T, b1 = ((last + 1) * G - 1) / f.T;
    f.nq_max = std::max<int>(f.nq_max, (int)(b1 - b0 + 1));
  }
  return f;
}

}  // namespace

namespace nvfp4v {
namespace passk {

int flow_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t H, int64_t I,
              const uint16_t *h0, int64_t m, const PassWs &w, uint16_t *h_out, uint16_t *trace,
              hipStream_t stream) {
  const int mb = (int)((m + 15) / 16);
  FlowConfig cfg;
  if (!pick_flow(mb, &cfg)) return NVFP4V_E_M_RANGE;
  const size_t lds = flow_lds_bytes(cfg);
  hipError_t e = hipFuncSetAttribute((const void *)cfg.kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return hip_status(ctx, e);
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)cfg.kern, (cfg.wc + 1) * 64, lds);
  if (e != hipSuccess) return hip_status(ctx, e);
  if (per_cu < 1) return NVFP4V_E_HIP;
  const int grid = ctx->num_cus;
  const int rt_per_block = cfg.wc * cfg.r;
  Layout ls[4];
  if (!make_layout(3 * H, H, &ls[0]) || !make_layout(H, H, &ls[1]) || !make_layout(2 * I, H, &ls[2]) ||
      !make_layout(H, I, &ls[3]))
    return NVFP4V_E_SHAPE;
  PassArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = (int)m;
  a.H = (int)H;
  a.last_layer = n_layers - 1;
  for (int j = 0; j < 4; ++j) {
    if (ls[j].bytes() > (size_t)0x7FFF0000) return NVFP4V_E_SHAPE;  // 32-bit buffer offsets
    a.ph[j].N = (int)ls[j].n;
    a.ph[j].nrt = (int)ls[j].nrt;
    a.ph[j].nkt = (int)ls[j].nkt;
    a.fs[j] = flow_shape(ls[j].nrt, ls[j].nkt, rt_per_block, grid);
    const FlowShape &f = a.fs[j];
    // partial tiles: (row block, piece, consumer wave) -> R x MB tiles of 256 floats
    const size_t part_need = (size_t)f.nrb * f.nq_max * cfg.wc * cfg.r * mb * 256;
    if (part_need > ctx->partial_floats || (size_t)f.nrb * cfg.wc > ctx->n_counters) return NVFP4V_E_WORKSPACE;
  }
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
  a.timeline = ctx->pass_timeline;
  ctx->last_pass_grid = grid;
  ctx->last_pass_phases = 4 * n_layers;
  if (fault_injected()) return NVFP4V_E_FAULT;

  int rc = launch_pack_act(ctx, h0, m, H, w.act0, stream, ctx->pass_sync);
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
    e = hipLaunchCooperativeKernel((const void *)cfg.kern, dim3((unsigned)grid), dim3((cfg.wc + 1) * 64), args,
                                   (unsigned)lds, stream);
    rc = hip_status(ctx, e);
  }
  return rc;
}

}  // namespace passk
}  // namespace nvfp4v
