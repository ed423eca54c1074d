// Declarations shared by the persistent pass kernel (pass.hip: one grid
// barrier per phase with a register ring per wave) and the chained launches:
// the pass workspace, the kernel arguments, the grid barrier and the fused
// epilogue of each phase. The stack and its glue are described in pass.hip.
#pragma once

#include "gemm_device.h"

namespace nvfp4v {
namespace passk {

using namespace nvfp4v::dev;

constexpr int LAYERS_PER_LAUNCH = 32;
constexpr uint64_t BARRIER_TIMEOUT_TICKS = 200000000ull;  // 2 s of the 100 MHz real-time clock

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// Workspace: the fp32 outputs of one layer (the last layer's are kept), then one
// block of packed activations per layer and phase (each phase reads a buffer
// of its own), then the packed h of the layer after the last one. Each block
// holds the bf16 copy and, act16 bytes after it, the fp16 copy.
// ---------------------------------------------------------------------------
struct PassWs {
  float *C[4];          // qkv [M][3H], o [M][H], gu [M][2I], d [M][H]
  uint8_t *act0;        // packed activations of layer 0, phase 0
  size_t layer_stride;  // bytes between the activation blocks of two layers
  size_t act_off[4];    // offset of phase j's input within a layer's block
  size_t act_bytes[4];  // one copy
  size_t act16[4];      // from the bf16 copy to the fp16 copy
  int64_t trace_m;      // rows of the trace's [layer][rows][H] layout (the pass's M, or
                        // the whole call's M when this pass is one block of its rows)
};

inline size_t pass_ws_layout(int64_t m, int64_t H, int64_t I, int n_layers, uint8_t *base, PassWs *w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w->C[0] = (float *)take((size_t)m * 3 * H * 4);
  w->C[1] = (float *)take((size_t)m * H * 4);
  w->C[2] = (float *)take((size_t)m * 2 * I * 4);
  w->C[3] = (float *)take((size_t)m * H * 4);
  w->act_bytes[0] = act_copy_bytes(m, H);  // h
  w->act_bytes[1] = act_copy_bytes(m, H);  // o_in
  w->act_bytes[2] = act_copy_bytes(m, H);  // g_in
  w->act_bytes[3] = act_copy_bytes(m, I);  // d_in
  size_t stride = 0;
  for (int j = 0; j < 4; ++j) {
    w->act_off[j] = stride;
    w->act16[j] = align256(w->act_bytes[j]);
    stride += 2 * w->act16[j];
  }
  w->layer_stride = stride;
  w->act0 = base ? base + off : nullptr;
  off += stride * (size_t)n_layers + 2 * w->act16[0];
  w->trace_m = m;
  return off;
}

// ---------------------------------------------------------------------------
// Persistent kernels.
// ---------------------------------------------------------------------------
// Work of one phase on a grid of G work-groups, in row blocks of R row tiles.
// Rounds 0..full-1: work-group g owns row block g + G * round over all of K.
// The `rem` row blocks left over are each cut into q pieces along K; piece
// g (g < rem * q) goes to work-group g and is processed last, its partial sums
// combined by whichever work-group finishes the row block's last piece.
struct PhaseShape {
  int N, nrt, nkt;
  int full, rem, q;
  int rows_rem;  // rem * R * 16: rows covered by the split row blocks
};

struct PassArgs {
  int n_layers;    // layers in this launch (<= LAYERS_PER_LAUNCH)
  int M;
  int layer0;      // index of this launch's first layer in the whole stack
  int last_layer;  // index of the stack's last layer
  PhaseShape ph[4];
  const uint8_t *w[LAYERS_PER_LAUNCH][4];
  float ts[LAYERS_PER_LAUNCH][4];
  float cst[4];  // glue constants: H^-1/2, H^-1/2, (2H)^-1/2, I^-1/2
  int H;
  uint8_t *act0;
  size_t layer_stride;
  size_t act_off[4];
  int act_bytes[4];
  float *C[4];
  uint16_t *h_out, *trace;
  int trace_m;  // rows of the trace's [layer][rows][H] layout
  float *part;
  unsigned *counters;
  unsigned *sync;  // barrier words (SYNC_* offsets)
  uint64_t *timeline;  // optional: [phase][work-group][2] real-time clock stamps
  int phase0;          // index of this launch's first phase in the timeline
};

// Barrier words, each on its own 256-byte line so arrivals and polls do not
// contend for one line: the release generation, the count of finished groups,
// the error flag, the count of work-groups that finished the launch, and one
// arrival counter per group of work-groups.
constexpr int SYNC_RELEASE = 0, SYNC_TOP = 64, SYNC_ERROR = 128, SYNC_DONE = 192, SYNC_GROUP0 = 256;
constexpr int BARRIER_GROUPS = 16;
constexpr int SYNC_WORDS = SYNC_GROUP0 + 64 * BARRIER_GROUPS;
static_assert(SYNC_WORDS == PASS_SYNC_WORDS, "barrier block size");

// Work-group barrier that orders LDS only: waits for this wave's LDS
// operations, not for its loads in flight (a fence before s_barrier would
// wait for every outstanding global load too, emptying the prefetch ring).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left open
  asm volatile("s_barrier" ::: "memory");
}

// Arrival at the grid barrier (thread 0 of the work-group, after every wave's
// stores of the phase have completed): work-group w arrives at the counter of
// group w % 16; the last arrival of a group arrives at the top counter, and
// the last group publishes generation `gen`.
__device__ inline void barrier_arrive(unsigned *sync, unsigned gen) {
  const unsigned g = blockIdx.x % BARRIER_GROUPS;
  const unsigned gsize = gridDim.x / BARRIER_GROUPS + (g < gridDim.x % BARRIER_GROUPS ? 1u : 0u);
  const unsigned old =
      __hip_atomic_fetch_add(&sync[SYNC_GROUP0 + 64 * g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (old + 1 == gen * gsize) {
    const unsigned groups = gridDim.x < BARRIER_GROUPS ? gridDim.x : BARRIER_GROUPS;
    const unsigned t =
        __hip_atomic_fetch_add(&sync[SYNC_TOP], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (t + 1 == gen * groups)
      __hip_atomic_store(&sync[SYNC_RELEASE], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

// Wait for generation `gen` (thread 0); false after the 2 s bound or when
// another work-group has already given up.
__device__ inline bool barrier_wait(unsigned *sync, unsigned gen) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(&sync[SYNC_RELEASE], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < gen) {
    __builtin_amdgcn_s_sleep(1);
    if (__hip_atomic_load(&sync[SYNC_ERROR], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > BARRIER_TIMEOUT_TICKS) {
      // The error word keeps the first site that gave up (1: a grid barrier).
      unsigned zero = 0;
      (void)__hip_atomic_compare_exchange_strong(&sync[SYNC_ERROR], &zero, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_SYSTEM);
      return false;
    }
  }
  return true;
}

// GEMM arguments and fused epilogue of phase p (the glue that feeds phase p+1).
__device__ inline GemmArgs phase_gemm(const PassArgs &a, int p) {
  const int l = p >> 2, j = p & 3;
  const int gl = a.layer0 + l;
  uint8_t *blk = a.act0 + (size_t)l * a.layer_stride;
  const PhaseShape &ps = a.ph[j];
  GemmArgs g;
  g.act = blk + a.act_off[j];
  g.M = a.M;
  g.act_bytes = a.act_bytes[j];
  g.W = a.w[l][j];
  g.N = ps.N;
  g.nrt = ps.nrt;
  g.nkt = ps.nkt;
  g.kts_per_split = ps.nkt;
  g.ksplit = 1;
  g.ts = a.ts[l][j];
  g.C = a.C[j];
  g.part = a.part;
  g.counters = a.counters;
  Epilogue &e = g.epi;
  e.c = a.cst[j];
  e.write_c = gl == a.last_layer ? 1 : 0;  // only the last layer's fp32 outputs are kept
  if (j == 0) {
    e.mode = EPI_SCALE, e.col0 = 2 * a.H, e.col1 = 3 * a.H, e.act = blk + a.act_off[1];
  } else if (j == 1) {
    e.mode = EPI_SCALE, e.col0 = 0, e.col1 = a.H, e.act = blk + a.act_off[2];
  } else if (j == 2) {
    e.mode = EPI_PAIR, e.act = blk + a.act_off[3];
  } else {
    e.mode = EPI_SCALE, e.col0 = 0, e.col1 = a.H;
    e.act = blk + a.layer_stride + a.act_off[0];  // next layer's input
    e.rm0 = gl == a.last_layer ? a.h_out : nullptr;
    e.rm1 = a.trace ? a.trace + (size_t)gl * a.trace_m * a.H : nullptr;
  }
  return g;
}

}  // namespace passk
}  // namespace nvfp4v
