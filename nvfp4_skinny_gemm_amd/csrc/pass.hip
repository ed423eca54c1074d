// The full verify pass: every linear layer of a dense layer stack applied to
// the M rows of a draft tree, chained layer to layer (TandemLLM manual, "What
// TandemLLM is", 1.2 "Two levers": one forward pass checks all guesses and
// reads the same weights whatever the row count).
//
// The pages give neither the layer shapes nor the non-GEMM operations, so the
// stack is a uniform stand-in: per layer, a fused q|k|v projection
// [3H x H], o [H x H], a fused gate|up projection [2I x H] (gate and up rows
// interleaved in 16-row tiles) and down [H x I], joined by elementwise glue
// that keeps activations O(1) (no reductions, no activation function, since the
// pages name none). The glue runs in the epilogue of the GEMM that produces
// its input:
//   qkv = h Wqkv^T;               o_in = bf16(v * H^-1/2)   (one-key attention)
//   o   = o_in Wo^T;              g_in = bf16(o * H^-1/2)
//   gu  = g_in Wgu^T;             d_in = bf16(gate * (2H)^-1/2 + up * (2H)^-1/2)
//   d   = d_in Wd^T;              h'   = bf16(d * I^-1/2)
// Every map is linear, so the activations' RMS stays O(1) over the whole stack
// (a product of gate and up would square it at every layer). Each glue value
// is one fp32 product, or two products and a sum without fused multiply-add,
// rounded to bf16 (nearest even).
//
// Execution: one persistent, cooperatively launched kernel runs up to 32
// layers (128 GEMM phases). Its work-groups take the units of a phase in turn
// (unit u -> row block u % grid_x, k-split u / grid_x; the same unit code as
// the per-call GEMM) and meet at a grid barrier before the next phase, whose
// input the previous phase's epilogues wrote. That removes the per-launch ramp
// and drain of 4 kernels per layer. Coherence across the dies' L2 caches
// without fences: the epilogues store the next phase's activations with
// system-coherent (write-through) stores, every phase reads its activations
// from a buffer no other phase of the launch uses (so no L2 can hold a stale
// copy of it; kernel boundaries invalidate the L2s), and the barrier counter
// is a system-scope atomic. The barrier wait is bounded: after 2 s it sets an
// error flag and the kernel ends, so a broken launch cannot hang the GPU.
#include <hip/hip_bf16.h>

#include <algorithm>
#include <cstdlib>
#include <cmath>

#include "pass_common.h"

using namespace nvfp4v;
using namespace nvfp4v::dev;
using namespace nvfp4v::passk;

namespace {

__device__ inline uint16_t to_bf16_bits(float x) {
  const __hip_bfloat16 b = __float2bfloat16(x);
  uint16_t u;
  __builtin_memcpy(&u, &b, 2);
  return u;
}

// out[r][j] = bf16(x[r * ldx + j] * c), r < rows, j < cols; out is dense.
__global__ void k_glue_scale(const float *__restrict__ x, int64_t ldx, int64_t rows, int64_t cols,
                             float c, uint16_t *__restrict__ out) {
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, j = i - r * cols;
    const float p = x[r * ldx + j] * c;
    out[i] = to_bf16_bits(p);
  }
}

// out[r][j] = bf16(x[r][j] * c + y[r][j] * c), the sum not fused with a product
__global__ void k_glue_sum(const float *__restrict__ x, int64_t ldx, const float *__restrict__ y,
                           int64_t ldy, int64_t rows, int64_t cols, float c,
                           uint16_t *__restrict__ out) {
#pragma clang fp contract(off)
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, j = i - r * cols;
    const float px = x[r * ldx + j] * c;
    const float py = y[r * ldy + j] * c;
    out[i] = to_bf16_bits(px + py);
  }
}

// Zero the last k-tile of the packed-activation blocks whose K is not a
// multiple of 256, for every layer (and the block after the last layer), in
// both copies: the epilogues write only the columns below K, while the GEMMs
// read whole k-tiles (the padded weights there are zero, but zero times a
// stale NaN is not). Block (l, j) starts at l * stride + off[j], its fp16 copy
// act16[j] bytes later; the tail is `tail[j]` bytes at tail_off[j] within a
// copy (tail[j] == 0: nothing to zero).
struct TailArgs {
  uint8_t *act0;
  size_t stride;
  size_t off[4], tail_off[4], act16[4];
  int tail[4];
  int layers;  // blocks of layers 0..layers-1 (all four), then block 0 of layer `layers`
};

__global__ void k_zero_tails(TailArgs t) {
  const int l = blockIdx.y, j = blockIdx.z;
  if (l == t.layers && j != 0) return;
  const int n16 = t.tail[j] / 16;
  uint8_t *blk = t.act0 + (size_t)l * t.stride + t.off[j] + t.tail_off[j];
  uint4 *dst = reinterpret_cast<uint4 *>(blk);
  uint4 *dst16 = reinterpret_cast<uint4 *>(blk + t.act16[j]);
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += gridDim.x * blockDim.x) {
    dst[i] = make_uint4(0u, 0u, 0u, 0u);
    dst16[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

unsigned glue_grid(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return (unsigned)(g < 2048 ? (g > 0 ? g : 1) : 2048);
}

// ---------------------------------------------------------------------------
// The persistent kernel.
// ---------------------------------------------------------------------------
// One work item of a wave: R row tiles x one k-tile of a task (a row block, or
// a piece of one) of phase p. A task whose k-range gives this wave no k-tile
// still yields one empty item (its loads return zeros) so that every wave
// takes part in the task's reduction.
struct Item {
  int p;     // phase index within the launch (4 * layer + projection)
  int task;  // index within the work-group's tasks of phase p
  int kt, kend;
  int rb;    // row block of the task
};

// The task's pieces and piece index (q = 1: a whole row block).
__device__ inline int task_count(const PhaseShape &ps, int g, int G) {
  return ps.full + (g < ps.rem * ps.q ? 1 : 0);
}

// Task order within a phase: the K-split piece (if the work-group has one)
// first, so that its slower flush overlaps the streaming of the whole row
// blocks instead of delaying the phase's end; then the whole row blocks.
__device__ inline bool task_is_piece(const PhaseShape &ps, int task, int g) {
  return task == 0 && g < ps.rem * ps.q;
}

// The task's pieces and piece index (q = 1: a whole row block).
__device__ inline void task_split(const PhaseShape &ps, const Item &it, int g, int *q, int *s) {
  if (task_is_piece(ps, it.task, g)) {
    *q = ps.q, *s = g % ps.q;
  } else {
    *q = 1, *s = 0;
  }
}

// Point `it` at the first item of task it.task of phase it.p, moving on to the
// next phase while the work-group has no task left; it.p == np at the end.
__device__ inline void seek(Item &it, const PassArgs &a, int np, int g, int G, int wave) {
  while (it.p < np) {
    const PhaseShape &ps = a.ph[it.p & 3];
    if (it.task < task_count(ps, g, G)) {
      int ka = 0, kb = ps.nkt;
      if (task_is_piece(ps, it.task, g)) {
        const int s = g % ps.q;
        it.rb = ps.full * G + g / ps.q;
        ka = (int)((int64_t)ps.nkt * s / ps.q);
        kb = (int)((int64_t)ps.nkt * (s + 1) / ps.q);
      } else {
        const int unit = it.task - (g < ps.rem * ps.q ? 1 : 0);
        it.rb = g + G * unit;
      }
      const int len = kb - ka;
      it.kt = ka + (len * wave) / WG_WAVES;
      it.kend = ka + (len * (wave + 1)) / WG_WAVES;
      return;
    }
    ++it.p;
    it.task = 0;
  }
}

__device__ inline void advance(Item &it, const PassArgs &a, int np, int g, int G, int wave) {
  if (it.kt + 1 < it.kend) {
    ++it.kt;
    return;
  }
  ++it.task;
  seek(it, a, np, g, G, wave);
}

__device__ inline bool last_of_task(const Item &it) { return it.kt + 1 >= it.kend; }

// Weight and activation loads of item `it` (zeros past the launch's items, for
// an empty item, or for row tiles past the matrix).
template <int R>
__device__ inline void load_item_w(WTile (&w)[R], const Item &it, const PassArgs &a, int np, int lane) {
  const bool valid = it.p < np;
  const int p = valid ? it.p : 0;
  const PhaseShape &ps = a.ph[p & 3];
  const int stripe = ps.nkt * TILE_BYTES;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void *)a.w[p >> 2][p & 3], (short)0, ps.nrt * stripe, RAW_BUFFER_FLAGS);
  const bool real = valid && it.kt < it.kend;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = it.rb * R + r;
    const int base = (real && rt < ps.nrt) ? rt * stripe + it.kt * TILE_BYTES : OOB;
    // Default cache policy: with the non-temporal hint of the per-call GEMM
    // this kernel measures 4 % slower (5.75 against 5.52 ms per pass).
    const auto c0 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + lane * 16, 0, 0);
    const auto c1 = __builtin_amdgcn_raw_buffer_load_b128(rs, base + CODE_HALF_BYTES + lane * 16, 0, 0);
    const auto sc = __builtin_amdgcn_raw_buffer_load_b32(rs, base + SCALE_OFFSET + lane * 4, 0, 0);
    __builtin_memcpy(&w[r].c[0], &c0, 16);
    __builtin_memcpy(&w[r].c[1], &c1, 16);
    w[r].s = (uint32_t)sc;
  }
}

template <int MB>
__device__ inline void load_item_a(bf16x8 (&b)[MB][8], const Item &it, const PassArgs &a, int np,
                                   bool ready, int lane) {
  const bool valid = it.p < np;
  const int p = valid ? it.p : 0;
  const int j = p & 3;
  const uint8_t *act = a.act0 + (size_t)(p >> 2) * a.layer_stride + a.act_off[j];
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)act, (short)0, a.act_bytes[j], RAW_BUFFER_FLAGS);
  load_afrag<MB>(b, ra, it.kt, ready && valid && it.kt < it.kend, a.M, lane);
}

// End of a task for the whole work-group: sum the four waves' tiles (wave
// order) in LDS buffer `red`, then either run the epilogue (a whole row block)
// or publish this piece's partial sums; the work-group holding the last piece
// of a row block sums the pieces in piece order and runs the epilogue.
// `ticket` is an LDS word. Leaves acc zeroed.
template <int MB, int R>
__device__ inline void flush_task(const PassArgs &a, const Item &it, f32x4 (&acc)[R][MB], f32x4 *red,
                                  unsigned *ticket, int tid, int lane, int wave) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      red[((wave * R + r) * MB + mb) * 64 + lane] = acc[r][mb];
      acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  lds_barrier();
  const GemmArgs g = phase_gemm(a, it.p);
  const PhaseShape &ps = a.ph[it.p & 3];
  const int rt0 = it.rb * R;
  int nq, sq;
  task_split(ps, it, (int)blockIdx.x, &nq, &sq);
  if (nq == 1) {
    epilogue<MB, R>(red, WG_WAVES, tid, a.M, g.N, g.nrt, rt0, g.ts, g.C, g.epi);
    return;
  }
  constexpr int ITEMS = R * MB * 64;
  const int lrb = it.rb - ps.full * (int)gridDim.x;  // index among the split row blocks
  const int M = a.M;
  for (int i = tid; i < ITEMS; i += WG_THREADS) {
    const int r = i / (MB * 64), mb = (i / 64) % MB, l = i & 63;
    f32x4 v = red[((0 * R + r) * MB + mb) * 64 + l];
#pragma unroll
    for (int wv = 1; wv < WG_WAVES; ++wv) v += red[((wv * R + r) * MB + mb) * 64 + l];
    const int m = mb * 16 + (l & 15), rt = rt0 + r;
    if (m >= M || rt >= ps.nrt) continue;
    float *dst = a.part + ((size_t)sq * M + m) * ps.rows_rem + (size_t)(lrb * R + r) * ROWS_PER_TILE +
                 4 * (l >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) __hip_atomic_store(dst + e, v[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  // The partial sums have reached memory once this wave's counters drain.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if (tid == 0)
    *ticket = __hip_atomic_fetch_add(&a.counters[lrb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  lds_barrier();
  const bool last = *ticket == (unsigned)(nq - 1);
  if (!last) return;
  for (int i = tid; i < ITEMS; i += WG_THREADS) {
    const int r = i / (MB * 64), mb = (i / 64) % MB, l = i & 63;
    const int m = mb * 16 + (l & 15), rt = rt0 + r;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    if (m < M && rt < ps.nrt) {
      const float *src = a.part + (size_t)m * ps.rows_rem + (size_t)(lrb * R + r) * ROWS_PER_TILE + 4 * (l >> 4);
      for (int s = 0; s < nq; ++s) {
        const float *ps_src = src + (size_t)s * M * ps.rows_rem;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] += __hip_atomic_load(ps_src + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    red[((0 * R + r) * MB + mb) * 64 + l] = v;  // slot of wave 0, read back by other threads
  }
  lds_barrier();
  if (tid == 0) __hip_atomic_store(&a.counters[lrb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  epilogue<MB, R>(red, 1, tid, a.M, g.N, g.nrt, rt0, g.ts, g.C, g.epi);
}

// Every wave streams its items through a two-deep ring (weights and
// activations of items t+1 and t+2 in flight while item t is computed) that
// runs on across task and phase boundaries: the next phase's weights are
// requested before the grid barrier, only its activations wait for it.
template <int MB, int R>
constexpr int pass_waves_per_simd() {
  return (MB == 1 && R <= 2) ? 3 : 2;
}

template <int MB, int R>
__global__ __launch_bounds__(WG_THREADS) __attribute__((amdgpu_waves_per_eu(pass_waves_per_simd<MB, R>())))
void k_pass(PassArgs a) {
  extern __shared__ __align__(16) f32x4 lds[];
  constexpr int RED = WG_WAVES * R * MB * 64;  // f32x4 per reduction buffer
  // s_waitcnt operand: vmcnt = the loads of one ring slot, lgkmcnt/expcnt open.
  constexpr int SLOT_LOADS = 3 * R + 8 * MB;
  constexpr int VMCNT_STORES = 0x0f70 | (SLOT_LOADS & 15) | ((SLOT_LOADS >> 4) << 14);
  unsigned *words = reinterpret_cast<unsigned *>(lds + 2 * RED);  // ticket, barrier flag
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.x, G = gridDim.x;
  const int np = 4 * a.n_layers;

  f32x4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Item it0, it1, it2;  // items t, t+1, t+2
  it0.p = 0, it0.task = 0;
  seek(it0, a, np, g, G, wave);
  it1 = it0;
  if (it1.p < np) advance(it1, a, np, g, G, wave);
  it2 = it1;
  if (it2.p < np) advance(it2, a, np, g, G, wave);

  int phase = 0;      // barriers passed
  int nflush = 0;     // tasks flushed (selects the reduction buffer)
  bool ok = true;
  auto stamp_phase = [&](int p, int which) {
    if (a.timeline && tid == 0 && g < PASS_TIMELINE_WGS && a.phase0 + p < (int)PASS_TIMELINE_PHASES)
      a.timeline[((size_t)(a.phase0 + p) * PASS_TIMELINE_WGS + g) * 2 + which] = __builtin_amdgcn_s_memrealtime();
  };

  // Move to phase `target` (one grid barrier per phase boundary). Every wave
  // has waited for its stores of the finished phase before calling; thread 0
  // arrives and waits, the other waves wait at the work-group barrier with
  // their prefetched weights still in flight.
  auto cross = [&](int target) {
    while (phase < target && ok) {
      stamp_phase(phase, 1);
      lds_barrier();
      if (tid == 0) {
        barrier_arrive(a.sync, (unsigned)(phase + 1));
        words[1] = barrier_wait(a.sync, (unsigned)(phase + 1)) ? 1u : 0u;
      }
      lds_barrier();
      ok = words[1] != 0;
      ++phase;
      stamp_phase(phase, 0);
    }
  };

  stamp_phase(0, 0);
  if (it0.p >= np) {
    __builtin_amdgcn_s_waitcnt(0);
    cross(np - 1);
  } else {
    cross(it0.p);
    WTile w0[R], w1[R];
    bf16x8 a0[MB][8], a1[MB][8];
    load_item_w<R>(w0, it0, a, np, lane);
    load_item_a<MB>(a0, it0, a, np, true, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_item_w<R>(w1, it1, a, np, lane);
    load_item_a<MB>(a1, it1, a, np, it1.p == phase, lane);
    __builtin_amdgcn_sched_barrier(0);

// One step: compute item t from ring slot (W, A), flush its task if it was the
// task's last item, refill the slot with item t+2, and cross to item t+1's
// phase if that is a new one. Every step issues the same loads in the same
// order (activations the barrier still gates are requested at an offset that
// returns zeros), and a crossing re-issues the slot's loads after item t+1's
// activations, so the compiler's wait counts hold on every path: item t+1
// waits only for its own loads, with item t+2's still in flight. The loop
// body runs both steps unconditionally and leaves only at its end (an early
// exit would give the structurised control flow a path that skips a step, and
// the wait counts would have to cover it); a step past the last item computes
// on zeros and neither flushes nor crosses.
#define NVFP4V_PASS_STEP(W, A, WO, AO)                                                       \
  {                                                                                           \
    _Pragma("unroll") for (int r = 0; r < R; ++r) compute_wtile<MB, false>(W[r], A, acc[r]); \
    if (it0.p < np && last_of_task(it0)) {                                                    \
      flush_task<MB, R>(a, it0, acc, lds + (nflush & 1) * RED, words, tid, lane, wave);      \
      ++nflush;                                                                               \
    }                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    load_item_w<R>(W, it2, a, np, lane);                                                      \
    load_item_a<MB>(A, it2, a, np, it2.p == phase, lane);                                     \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    it0 = it1;                                                                                \
    it1 = it2;                                                                                \
    if (it2.p < np) advance(it2, a, np, g, G, wave);                                          \
    if (it0.p < np && it0.p != phase) {                                                       \
      /* this wave's epilogue stores precede the slot's loads just issued */                 \
      __builtin_amdgcn_s_waitcnt(VMCNT_STORES);                                               \
      cross(it0.p);                                                                           \
      if (!ok) it0.p = it1.p = it2.p = np;                                                    \
      load_item_a<MB>(AO, it0, a, np, true, lane);                                            \
      __builtin_amdgcn_sched_barrier(0);                                                      \
      load_item_w<R>(W, it1, a, np, lane);                                                    \
      load_item_a<MB>(A, it1, a, np, it1.p == phase, lane);                                   \
      __builtin_amdgcn_sched_barrier(0);                                                      \
    }                                                                                         \
  }

    do {
      NVFP4V_PASS_STEP(w0, a0, w1, a1)
      NVFP4V_PASS_STEP(w1, a1, w0, a0)
    } while (it0.p < np);
#undef NVFP4V_PASS_STEP
    // Phases after this work-group's last item (if any) still need its barrier arrivals.
    __builtin_amdgcn_s_waitcnt(0);
    if (ok) cross(np - 1);
  }
  stamp_phase(np - 1, 1);

  // The last work-group to finish resets the barrier words for the next launch.
  __builtin_amdgcn_s_waitcnt(0);
  lds_barrier();
  if (tid == 0) {
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

typedef void (*PassKernel)(PassArgs);

// Row tiles per wave item: 4 at one row block of activations (each activation
// fragment then serves 4 weight tiles), 2 at two (the ring of two row blocks of
// fragments leaves no room for more). NVFP4V_PASS_R overrides it.
PassKernel pick_pass_kernel(int mb, int *r, int *wgs_per_cu) {
  const char *renv = std::getenv("NVFP4V_PASS_R");
  int want = mb == 1 ? 4 : 2;
  if (renv && (std::atoi(renv) == 2 || std::atoi(renv) == 4)) want = std::atoi(renv);
  *r = want;
  switch (mb * 16 + want) {
    case 1 * 16 + 2: *wgs_per_cu = pass_waves_per_simd<1, 2>(); return k_pass<1, 2>;
    case 1 * 16 + 4: *wgs_per_cu = pass_waves_per_simd<1, 4>(); return k_pass<1, 4>;
    case 2 * 16 + 2: *wgs_per_cu = pass_waves_per_simd<2, 2>(); return k_pass<2, 2>;
    case 2 * 16 + 4: *wgs_per_cu = pass_waves_per_simd<2, 4>(); return k_pass<2, 4>;
    default: return nullptr;
  }
}

// LDS of k_pass: two reduction buffers, the ticket and the barrier flag.
size_t pass_lds_bytes(int mb, int r) { return (size_t)2 * WG_WAVES * r * mb * 64 * 16 + 16; }

// Split a phase of nrt row tiles x nkt k-tiles over G work-groups (see
// PhaseShape): whole row blocks first, then the remainder cut along K into at
// most G pieces of at least 4 k-tiles (one per wave) where K allows.
PhaseShape split_phase(int64_t n, int64_t nrt, int64_t nkt, int G, int R) {
  PhaseShape ps;
  ps.N = (int)n;
  ps.nrt = (int)nrt;
  ps.nkt = (int)nkt;
  const int nrb = (int)((nrt + R - 1) / R);
  ps.full = nrb / G;
  ps.rem = nrb - ps.full * G;
  ps.q = 1;
  if (ps.rem > 0) ps.q = std::max(1, std::min(G / ps.rem, (int)(nkt / WG_WAVES)));
  ps.rows_rem = ps.rem * R * ROWS_PER_TILE;
  return ps;
}

// The pass as four stream-ordered GEMM launches per layer. Each epilogue
// writes the next GEMM's packed activations into the same per-layer blocks
// the persistent kernel uses (the two schedules split K differently, so their
// fp32 sums can differ in the last bits).
int chain_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t H, int64_t I,
               const uint16_t *h0, int64_t m, const PassWs &w, uint16_t *h_out, uint16_t *trace,
               hipStream_t stream) {
  if (fault_injected()) return NVFP4V_E_FAULT;
  const float ch = (float)(1.0 / std::sqrt((double)H));
  const float c2h = (float)(1.0 / std::sqrt(2.0 * (double)H));
  const float ci = (float)(1.0 / std::sqrt((double)I));
  // The GEMMs compute from the fp16 copies (unless NVFP4V_F16=0), which the
  // packing kernel and the epilogues write beside the bf16 ones.
  const bool f16 = use_f16();
  const size_t x16[4] = {f16 ? w.act16[0] : 0, f16 ? w.act16[1] : 0, f16 ? w.act16[2] : 0, f16 ? w.act16[3] : 0};
  int rc = launch_pack_act(ctx, h0, m, H, w.act0, x16[0], stream);
  for (int l = 0; l < n_layers && rc == NVFP4V_OK; ++l) {
    const nvfp4v_layer &L = layers[l];
    uint8_t *blk = w.act0 + (size_t)l * w.layer_stride;
    uint8_t *a_h = blk + w.act_off[0], *a_o = blk + w.act_off[1];
    uint8_t *a_g = blk + w.act_off[2], *a_d = blk + w.act_off[3];
    uint8_t *a_next = blk + w.layer_stride + w.act_off[0];
    Epilogue e_o, e_g, e_d, e_h;
    e_o.mode = EPI_SCALE, e_o.col0 = (int)(2 * H), e_o.col1 = (int)(3 * H), e_o.c = ch, e_o.act = a_o;
    e_g.mode = EPI_SCALE, e_g.col0 = 0, e_g.col1 = (int)H, e_g.c = ch, e_g.act = a_g;
    e_d.mode = EPI_PAIR, e_d.c = c2h, e_d.act = a_d;
    e_h.mode = EPI_SCALE, e_h.col0 = 0, e_h.col1 = (int)H, e_h.c = ci, e_h.act = a_next;
    e_o.act16 = (int)x16[1], e_g.act16 = (int)x16[2], e_d.act16 = (int)x16[3], e_h.act16 = (int)x16[0];
    e_h.rm0 = (l == n_layers - 1) ? h_out : nullptr;
    e_h.rm1 = trace ? trace + (size_t)l * w.trace_m * H : nullptr;
    // Only the last layer's fp32 outputs are kept: earlier ones would be overwritten unread.
    e_o.write_c = e_g.write_c = e_d.write_c = e_h.write_c = (l == n_layers - 1) ? 1 : 0;
    rc = launch_gemm(ctx, a_h, x16[0], m, H, (const uint8_t *)L.qkv, 3 * H, L.ts_qkv, w.C[0], stream, e_o);
    if (!rc) rc = launch_gemm(ctx, a_o, x16[1], m, H, (const uint8_t *)L.o, H, L.ts_o, w.C[1], stream, e_g);
    if (!rc) rc = launch_gemm(ctx, a_g, x16[2], m, H, (const uint8_t *)L.gate_up, 2 * I, L.ts_gate_up, w.C[2], stream, e_d);
    if (!rc) rc = launch_gemm(ctx, a_d, x16[3], m, I, (const uint8_t *)L.down, H, L.ts_down, w.C[3], stream, e_h);
  }
  return rc;
}

}  // namespace

extern "C" int nvfp4v_glue_scale(nvfp4v_ctx *ctx, const float *x, int64_t ldx, int64_t rows,
                                 int64_t cols, float c, uint16_t *out, hipStream_t stream) {
  if (!ctx || !x || !out) return NVFP4V_E_INVALID_ARG;
  if (rows < 1 || cols < 1 || ldx < cols) return NVFP4V_E_SHAPE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  hipLaunchKernelGGL(k_glue_scale, dim3(glue_grid(rows * cols)), dim3(256), 0, stream, x, ldx, rows,
                     cols, c, out);
  return hip_status(ctx, hipGetLastError());
}

extern "C" int nvfp4v_glue_sum(nvfp4v_ctx *ctx, const float *x, int64_t ldx, const float *y,
                               int64_t ldy, int64_t rows, int64_t cols, float c, uint16_t *out,
                               hipStream_t stream) {
  if (!ctx || !x || !y || !out) return NVFP4V_E_INVALID_ARG;
  if (rows < 1 || cols < 1 || ldx < cols || ldy < cols) return NVFP4V_E_SHAPE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  hipLaunchKernelGGL(k_glue_sum, dim3(glue_grid(rows * cols)), dim3(256), 0, stream, x, ldx, y, ldy,
                     rows, cols, c, out);
  return hip_status(ctx, hipGetLastError());
}

// Workspace of a pass over m rows: one block of rows (at most CHUNK_M) after
// another, each laid out as pass_ws_layout lays out a pass of its rows.
static size_t rows_ws_bytes(int64_t m, int64_t hidden, int64_t inter, int n_layers, int64_t upto) {
  size_t total = 0;
  for (int64_t r0 = 0; r0 < m && r0 < upto; r0 += CHUNK_M) {
    PassWs w;
    total += align256(pass_ws_layout(std::min<int64_t>(CHUNK_M, m - r0), hidden, inter, n_layers, nullptr, &w));
  }
  return total;
}

extern "C" size_t nvfp4v_pass_workspace_bytes(int64_t m, int64_t hidden, int64_t inter,
                                              int n_layers) {
  if (m < 1 || m > NVFP4V_MAX_M || hidden < 16 || inter < 16 || n_layers < 1) return 0;
  if (hidden % 16 || inter % 16) return 0;
  return rows_ws_bytes(m, hidden, inter, n_layers, m);
}

extern "C" int nvfp4v_pass_status(nvfp4v_ctx *ctx) {
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  unsigned flag = 0;
  hipError_t e = hipMemcpy(&flag, ctx->pass_sync + SYNC_ERROR, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(ctx, e);
  return flag ? NVFP4V_E_TIMEOUT : NVFP4V_OK;
}

extern "C" int nvfp4v_pass_error_site(nvfp4v_ctx *ctx) {
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  unsigned site = 0;
  hipError_t e = hipMemcpy(&site, ctx->pass_sync + SYNC_ERROR, sizeof(unsigned), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(ctx, e);
  return (int)site;
}

// The pass over one block of at most CHUNK_M rows (arguments checked).
static int verify_pass_block(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t hidden,
                             int64_t inter, const uint16_t *h0, int64_t m, void *ws, uint16_t *h_out,
                             uint16_t *trace, int64_t trace_m, hipStream_t stream);

extern "C" int nvfp4v_verify_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers,
                                  int64_t hidden, int64_t inter, const uint16_t *h0, int64_t m,
                                  void *ws, size_t ws_bytes, uint16_t *h_out, uint16_t *trace,
                                  hipStream_t stream) {
  if (!ctx || !layers || !h0 || !ws || !h_out) return NVFP4V_E_INVALID_ARG;
  if (n_layers < 1) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  if (hidden < 16 || inter < 16 || hidden % 16 || inter % 16) return NVFP4V_E_SHAPE;
  Layout lq, lo, lg, ld;
  if (!make_layout(3 * hidden, hidden, &lq) || !make_layout(hidden, hidden, &lo) ||
      !make_layout(2 * inter, hidden, &lg) || !make_layout(hidden, inter, &ld))
    return NVFP4V_E_SHAPE;
  if (!aligned16(h0) || !aligned16(ws) || !aligned16(h_out) || (trace && !aligned16(trace)))
    return NVFP4V_E_ALIGN;
  for (int l = 0; l < n_layers; ++l)
    if (!layers[l].qkv || !layers[l].o || !layers[l].gate_up || !layers[l].down)
      return NVFP4V_E_INVALID_ARG;
  if (ws_bytes < rows_ws_bytes(m, hidden, inter, n_layers, m)) return NVFP4V_E_WORKSPACE;
  // Rows are independent through every GEMM and every glue step, so more
  // than CHUNK_M rows (several sequences' trees) run as one pass per block of
  // rows, each on its own part of the workspace.
  int rc = NVFP4V_OK;
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    uint8_t *wsb = (uint8_t *)ws + rows_ws_bytes(m, hidden, inter, n_layers, r0);
    rc = verify_pass_block(ctx, layers, n_layers, hidden, inter, h0 + r0 * hidden, mc, wsb,
                           h_out + r0 * hidden, trace ? trace + r0 * hidden : nullptr, m, stream);
  }
  return rc;
}

static int verify_pass_block(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers, int64_t hidden,
                             int64_t inter, const uint16_t *h0, int64_t m, void *ws, uint16_t *h_out,
                             uint16_t *trace, int64_t trace_m, hipStream_t stream) {
  Layout lq, lo, lg, ld;
  (void)make_layout(3 * hidden, hidden, &lq), (void)make_layout(hidden, hidden, &lo);
  (void)make_layout(2 * inter, hidden, &lg), (void)make_layout(hidden, inter, &ld);
  PassWs w;
  (void)pass_ws_layout(m, hidden, inter, n_layers, (uint8_t *)ws, &w);
  w.trace_m = trace_m;
  if (hidden % K_PER_TILE || inter % K_PER_TILE) {
    TailArgs t;
    t.act0 = w.act0;
    t.stride = w.layer_stride;
    t.layers = n_layers;
    const int mb = (int)((m + 15) / 16);
    const int64_t ks[4] = {hidden, hidden, hidden, inter};
    int most = 0;
    for (int j = 0; j < 4; ++j) {
      const int64_t nkt = (ks[j] + K_PER_TILE - 1) / K_PER_TILE;
      t.off[j] = w.act_off[j];
      t.act16[j] = w.act16[j];
      t.tail_off[j] = (size_t)(nkt - 1) * mb * 8 * ACT_FRAG_BYTES;
      t.tail[j] = ks[j] % K_PER_TILE ? mb * 8 * ACT_FRAG_BYTES : 0;
      most = std::max(most, t.tail[j]);
    }
    hipLaunchKernelGGL(k_zero_tails, dim3((unsigned)((most / 16 + 255) / 256), (unsigned)(n_layers + 1), 4),
                       dim3(256), 0, stream, t);
    const int rc = hip_status(ctx, hipGetLastError());
    if (rc) return rc;
  }
  if (ctx->pass_mode == NVFP4V_PASS_CHAIN) return chain_pass(ctx, layers, n_layers, hidden, inter, h0, m, w, h_out, trace, stream);

  const int mb = (int)((m + 15) / 16);
  int target_per_cu = 0, pr = 0;
  PassKernel kern = pick_pass_kernel(mb, &pr, &target_per_cu);
  // Rows beyond 32 keep the chained launches (the two-deep ring of 3-4 row
  // blocks of activations does not fit the registers of two waves per SIMD).
  if (!kern) return chain_pass(ctx, layers, n_layers, hidden, inter, h0, m, w, h_out, trace, stream);
  const size_t lds = pass_lds_bytes(mb, pr);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)kern, WG_THREADS, lds);
  if (e != hipSuccess) return hip_status(ctx, e);
  if (per_cu < 1) return NVFP4V_E_HIP;
  // One work-group per SIMD wave slot the kernel was compiled for (override:
  // NVFP4V_PASS_WGS=<work-groups per CU>, for measurements).
  const char *wenv = std::getenv("NVFP4V_PASS_WGS");
  if (wenv && std::atoi(wenv) > 0) target_per_cu = std::atoi(wenv);
  const int grid = std::min(per_cu, target_per_cu) * ctx->num_cus;
  PassArgs a;
  std::memset(&a, 0, sizeof(a));
  a.M = (int)m;
  a.H = (int)hidden;
  a.last_layer = n_layers - 1;
  const Layout *ls[4] = {&lq, &lo, &lg, &ld};
  for (int j = 0; j < 4; ++j) {
    if (ls[j]->bytes() > (size_t)0x7FFF0000) return NVFP4V_E_SHAPE;  // 32-bit buffer offsets
    a.ph[j] = split_phase(ls[j]->n, ls[j]->nrt, ls[j]->nkt, grid, pr);
    const PhaseShape &ps = a.ph[j];
    if (ps.rem > 0 && ps.q > 1) {
      const size_t part_need = (size_t)ps.q * (size_t)m * (size_t)ps.rows_rem;
      if (part_need > ctx->partial_floats || (size_t)ps.rem > ctx->n_counters) return NVFP4V_E_WORKSPACE;
    }
  }
  a.cst[0] = a.cst[1] = (float)(1.0 / std::sqrt((double)hidden));
  a.cst[2] = (float)(1.0 / std::sqrt(2.0 * (double)hidden));
  a.cst[3] = (float)(1.0 / std::sqrt((double)inter));
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

  // The persistent kernel computes from the bf16 copies only.
  int rc = launch_pack_act(ctx, h0, m, hidden, w.act0, 0, stream, ctx->pass_sync);
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
    e = hipLaunchCooperativeKernel((const void *)kern, dim3((unsigned)grid), dim3(WG_THREADS), args,
                                   (unsigned)lds, stream);
    rc = hip_status(ctx, e);
  }
  return rc;
}
