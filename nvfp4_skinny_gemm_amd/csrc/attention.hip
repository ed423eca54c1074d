// Tree-verify attention: one attention layer of the verify pass, for the M
// rows of one draft tree (the root token and the tree's nodes) against the
// committed context. The served model mixes Gated DeltaNet layers with
// attention layers (TandemLLM manual, "What TandemLLM is", 1.1 "The test
// environment"); the verify pass runs every row of the tree through each of
// them at once (1.2 "Two levers"), and its cost is measured per context length
// from 1k to 32k tokens (release post, the paragraph on what checking 8 to 32
// guesses costs).
//
// What is computed (fp32 on the device, bf16 inputs):
//   O[i][h] = sum_j softmax_j(scale * q_i,h . k_j) v_j
// over the positions j that row i sees: every context position 0..T-1 and the
// tree rows on its own path to the root (itself included), whose keys and
// values sit at positions T + row in the same cache. Query head h reads
// key/value head h / (Hq / Hkv).
//
// Like the verify GEMM, the layer streams bytes: each key/value head's cache
// is read once for all M rows, so the cost is the cache size over HBM
// bandwidth and is nearly flat in M. Design for gfx950:
//  * Caches are stored in MFMA fragment order, so every load is a 16-byte
//    lane load of one contiguous 1 KiB fragment: keys in blocks of 16
//    positions (lane = (d-group g, position i), 8 consecutive d), values
//    transposed in groups of 32 positions (lane = (g, d), the 8 positions
//    that lane g's slots of the P^T operand hold).
//  * S^T (positions x query columns) = K * Q^T and O^T (d x columns) =
//    V^T * P^T run on v_mfma_f32_16x16x32_bf16; the query columns are the
//    (query head of the group, row) pairs, 16 or 32 of them. P is split into
//    two bf16 terms (hi + lo), so the weights keep ~16 bits, not 8.
//  * Work: one work-group per (key/value head, chunk of positions); its four
//    waves take 32-position groups round-robin with an online softmax each,
//    merge in LDS in wave order, and publish the chunk's (max, sum, O) record.
//    The last work-group of a head to arrive (a ticket) merges the records in
//    chunk order and writes O. Every sum has a fixed order, so the result is
//    bitwise reproducible. Records cross XCDs through memory: system-scope
//    stores and loads, which leave the L2 out, and a ticket after the stores
//    are acknowledged (a device-scope fence instead writes back and invalidates
//    the whole L2 of the XCD; one per work-group cost ~70 us per call).
#include <hip/hip_bf16.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "gemm_device.h"

using namespace nvfp4v;
using namespace nvfp4v::dev;

namespace {

constexpr int HEAD_D = NVFP4V_ATTN_HEAD_DIM;  // 128
constexpr int GROUP_POS = 32;                 // positions per S^T pair / P^T operand
constexpr int ATTN_WAVES = 4;
constexpr int ATTN_THREADS = 64 * ATTN_WAVES;
constexpr int DBLK = HEAD_D / 16;  // 8 d-blocks of the O^T accumulators
constexpr int KSTEP = HEAD_D / 32;  // 4 MFMAs per S^T tile
// Cache policy bits sc0 sc1 (system scope) of the record stores and loads: the
// L2 of the writer's XCD is written through and the reader's is not consulted.
constexpr int SYSTEM_AUX = 17;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Record of one (head, chunk): per column max and sum, then O^T in the
// accumulator lane order [NB][DBLK][64 lanes][4].
template <int NB>
constexpr int record_floats() { return NB * 16 * 2 + NB * DBLK * 64 * 4; }

struct AttnArgs {
  const uint16_t *q;   // bf16 [M][Hq][D]
  const uint16_t *kc;  // key cache, fragment order
  const uint16_t *vc;  // value cache, fragment order
  float *o;            // fp32 [M][Hq][D]
  float *rec;          // [Hkv][nchunks] records
  unsigned *cnt;       // [Hkv] arrival tickets (zero between calls)
  int64_t cap;         // cache capacity in positions (multiple of 32)
  int T, M, hq, hkv, group, P, chunk, nchunks;
  int ncb;             // work-groups per (head, chunk), each NB column blocks of its own
  float scale;
  uint32_t vis[NVFP4V_ATTN_MAX_ROWS];  // bit j of vis[i]: row i sees tree row j
};

// Offsets (in bf16 elements) of a lane's 16 bytes in the caches.
__device__ inline size_t kfrag(const AttnArgs &a, int h, int64_t blk16, int s, int lane) {
  return ((((size_t)h * (size_t)(a.cap / 16) + (size_t)blk16) * KSTEP + s) * 64 + lane) * 8;
}
__device__ inline size_t vfrag(const AttnArgs &a, int h, int64_t grp32, int dblk, int lane) {
  return ((((size_t)h * (size_t)(a.cap / 32) + (size_t)grp32) * DBLK + dblk) * 64 + lane) * 8;
}

__device__ inline bf16x8 load16(const uint16_t *p) {
  const uint4 v = *reinterpret_cast<const uint4 *>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

template <int NB>
__global__ __launch_bounds__(ATTN_THREADS, 2) void k_tree_attn(AttnArgs a) {
  __shared__ float s_m[ATTN_WAVES][NB * 16];
  __shared__ float s_l[ATTN_WAVES][NB * 16];
  __shared__ f32x4 s_o[ATTN_WAVES][NB][DBLK][64];
  __shared__ unsigned s_last;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y, ci = blockIdx.x, z = blockIdx.z;
  const int col0 = z * NB * 16;  // this work-group's first query column
  const int hz = h * a.ncb + z;  // its record set and ticket
  const int g = lane >> 4, c16 = lane & 15;
  const int p0 = ci * a.chunk, p1 = min(a.P, p0 + a.chunk);
  const int ngroups = (p1 - p0 + GROUP_POS - 1) / GROUP_POS;
  const int ncols = a.group * a.M;

  // Query fragments (B operand of S^T): lane (g, c) holds q[row][8 consecutive d].
  bf16x8 qf[NB][KSTEP];
  int rowc[NB];  // query row of this lane's column, or -1 for a padding column
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int c = col0 + cb * 16 + c16;
    rowc[cb] = c < ncols ? c % a.M : -1;
    const int qh = h * a.group + (c < ncols ? c / a.M : 0);
#pragma unroll
    for (int s = 0; s < KSTEP; ++s) {
      if (c < ncols) {
        qf[cb][s] = load16(a.q + ((size_t)rowc[cb] * a.hq + qh) * HEAD_D + 32 * s + 8 * g);
      } else {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        __builtin_memcpy(&qf[cb][s], &z, 16);
      }
    }
  }

  float mrun[NB], lrun[NB];
  f32x4 oacc[NB][DBLK];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    mrun[cb] = -INFINITY;
    lrun[cb] = 0.f;
#pragma unroll
    for (int d = 0; d < DBLK; ++d) oacc[cb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Each wave walks its 32-position groups (gi = wave, wave + 4, ...) with the
  // keys and values of later groups requested as soon as a register set has
  // been consumed: its keys after the S^T products, its values after the P V
  // products. With one column block the wave keeps two register sets, so two
  // groups are in flight; with two it keeps one (registers). The groups are
  // processed in the same order either way.
  constexpr int SETS = NB == 1 ? 2 : 1;
  bf16x8 kf[SETS][2][KSTEP], vf[SETS][DBLK];
  auto pos_of = [&](int gi) { return p0 + gi * GROUP_POS; };
  auto load_k = [&](int set, int pb) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KSTEP; ++s) kf[set][t][s] = load16(a.kc + kfrag(a, h, pb / 16 + t, s, lane));
  };
  auto load_v = [&](int set, int pb) {
#pragma unroll
    for (int d = 0; d < DBLK; ++d) vf[set][d] = load16(a.vc + vfrag(a, h, pb / 32, d, lane));
  };
  // One group with register set `set`; then that set is refilled with group
  // gnext (if it exists).
  auto step = [&](int set, int gi, int gnext) {
    const int pbase = pos_of(gi);  // a multiple of 32
    const bool more = gnext < ngroups;
    f32x4 st[NB][2];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        st[cb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEP; ++s)
          st[cb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[set][t][s], qf[cb][s], st[cb][t], 0, 0, 0);
      }
    if (more) load_k(set, pos_of(gnext));

    if (pbase + GROUP_POS > a.P) {
      // Cache slots past the last position may hold anything (NaN included):
      // zero them, as a zero weight times NaN would still be NaN.
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int pos = pbase + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
        if (pos >= a.P) {
#pragma unroll
          for (int d = 0; d < DBLK; ++d) vf[set][d][j] = (__bf16)0.f;
        }
      }
    }

#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      // Lane (g, c) holds the scores of positions pbase + 16 t + 4 g + r.
      const int row = rowc[cb];
      const uint32_t vis = row >= 0 ? a.vis[row] : 0xFFFFFFFFu;
      float sc[8];
      bool ok[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = j >> 2, r = j & 3;
        const int pos = pbase + 16 * t + 4 * g + r;
        ok[j] = pos < a.T || (pos < a.P && ((vis >> (pos - a.T)) & 1u));
        sc[j] = ok[j] ? st[cb][t][r] * a.scale : -INFINITY;
        tmax = fmaxf(tmax, sc[j]);
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[cb], tmax);
      const float alpha = mnew == mrun[cb] ? 1.f : expf(mrun[cb] - mnew);
      mrun[cb] = mnew;
      bf16x8 phi, plo;
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = ok[j] ? expf(sc[j] - mnew) : 0.f;
        psum += p;
        const __bf16 hi = (__bf16)p;
        phi[j] = hi;
        plo[j] = (__bf16)(p - (float)hi);
      }
      lrun[cb] = lrun[cb] * alpha + psum;
#pragma unroll
      for (int d = 0; d < DBLK; ++d) {
        oacc[cb][d] *= alpha;
        oacc[cb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[set][d], phi, oacc[cb][d], 0, 0, 0);
        oacc[cb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[set][d], plo, oacc[cb][d], 0, 0, 0);
      }
    }
    if (more) load_v(set, pos_of(gnext));
  };

  constexpr int STRIDE = ATTN_WAVES * SETS;  // groups between two uses of one register set
#pragma unroll
  for (int sset = 0; sset < SETS; ++sset) {
    const int gi = wave + sset * ATTN_WAVES;
    if (gi < ngroups) {
      load_k(sset, pos_of(gi));
      load_v(sset, pos_of(gi));
    }
  }
  for (int gi = wave; gi < ngroups; gi += STRIDE) {
#pragma unroll
    for (int sset = 0; sset < SETS; ++sset) {
      const int gs = gi + sset * ATTN_WAVES;
      if (gs < ngroups) step(sset, gs, gs + STRIDE);
    }
  }

  // ---- merge the four waves in LDS (wave order) ----
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float l = lrun[cb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (g == 0) {
      s_m[wave][cb * 16 + c16] = mrun[cb];
      s_l[wave][cb * 16 + c16] = l;
    }
#pragma unroll
    for (int d = 0; d < DBLK; ++d) s_o[wave][cb][d][lane] = oacc[cb][d];
  }
  __syncthreads();

  // One chunk per head: this work-group's merge is the result.
  if (a.nchunks == 1) {
    for (int it = tid; it < NB * DBLK * 64; it += ATTN_THREADS) {
      const int cb = it / (DBLK * 64), d = (it / 64) % DBLK, ln = it & 63;
      const int cl = cb * 16 + (ln & 15), c = col0 + cl;
      if (c >= ncols) continue;
      float mx = -INFINITY;
      for (int w = 0; w < ATTN_WAVES; ++w) mx = fmaxf(mx, s_m[w][cl]);
      float l = 0.f;
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int w = 0; w < ATTN_WAVES; ++w) {
        if (s_m[w][cl] == -INFINITY) continue;
        const float f = expf(s_m[w][cl] - mx);
        l += s_l[w][cl] * f;
        v += s_o[w][cb][d][ln] * f;
      }
      const float inv = 1.f / l;
      const int row = c % a.M, qh = h * a.group + c / a.M;
      float *dst = a.o + ((size_t)row * a.hq + qh) * HEAD_D + d * 16 + 4 * (ln >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = v[r] * inv;
    }
    return;
  }

  // The chunk's record, through memory (system scope: sc0 sc1 stores).
  float *rec = a.rec + ((size_t)hz * a.nchunks + ci) * record_floats<NB>();
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.rec + (size_t)hz * a.nchunks * record_floats<NB>()), (short)0,
      (int)((size_t)a.nchunks * record_floats<NB>() * sizeof(float)), RAW_BUFFER_FLAGS);
  const int rbase = ci * record_floats<NB>() * (int)sizeof(float);  // this record, bytes
  if (tid < NB * 16) {
    float mx = -INFINITY;
    for (int w = 0; w < ATTN_WAVES; ++w) mx = fmaxf(mx, s_m[w][tid]);
    float l = 0.f;
    for (int w = 0; w < ATTN_WAVES; ++w)
      if (s_m[w][tid] != -INFINITY) l += s_l[w][tid] * expf(s_m[w][tid] - mx);
    __hip_atomic_store(rec + tid, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(rec + NB * 16 + tid, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  for (int it = tid; it < NB * DBLK * 64; it += ATTN_THREADS) {
    const int cb = it / (DBLK * 64), d = (it / 64) % DBLK, ln = it & 63;
    const int cl = cb * 16 + (ln & 15);
    float mx = -INFINITY;
    for (int w = 0; w < ATTN_WAVES; ++w) mx = fmaxf(mx, s_m[w][cl]);
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < ATTN_WAVES; ++w)
      if (s_m[w][cl] != -INFINITY) v += s_o[w][cb][d][ln] * expf(s_m[w][cl] - mx);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rr,
                                           rbase + (NB * 32 + it * 4) * (int)sizeof(float), 0, SYSTEM_AUX);
  }
  // Publish the record: every store acknowledged, then the ticket.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&a.cnt[hz], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    s_last = old == (unsigned)(a.nchunks - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- last arriver: merge the head's chunks in order and write O ----
  // Every record's maxima and sums into LDS first (independent loads, eight
  // per thread in flight), then each output element's chunk terms in batches
  // of eight loads, summed in chunk order.
  float *s_ml = reinterpret_cast<float *>(&s_o[0][0][0][0]);  // [nchunks][NB * 32]
  const int nml = a.nchunks * NB * 32;
  for (int base = tid; base < nml; base += ATTN_THREADS * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * ATTN_THREADS;
      const int k = idx / (NB * 32), j = idx % (NB * 32);
      v[u] = idx < nml ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                        rr, (k * record_floats<NB>() + j) * (int)sizeof(float), 0,
                                                        SYSTEM_AUX))
                       : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * ATTN_THREADS < nml) s_ml[base + u * ATTN_THREADS] = v[u];
  }
  __syncthreads();
  for (int it = tid; it < NB * DBLK * 64; it += ATTN_THREADS) {
    const int cb = it / (DBLK * 64), d = (it / 64) % DBLK, ln = it & 63;
    const int cl = cb * 16 + (ln & 15), c = col0 + cl;
    if (c >= ncols) continue;
    float mx = -INFINITY;
    for (int k = 0; k < a.nchunks; ++k) mx = fmaxf(mx, s_ml[k * NB * 32 + cl]);
    float l = 0.f;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < a.nchunks; k0 += 8) {
      f32x4 part[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        part[u] = k < a.nchunks ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                               rr, (k * record_floats<NB>() + NB * 32 + it * 4) *
                                                                       (int)sizeof(float),
                                                               0, SYSTEM_AUX))
                                : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        if (k >= a.nchunks) break;
        const float mk = s_ml[k * NB * 32 + cl];
        if (mk == -INFINITY) continue;
        const float f = expf(mk - mx);
        l += s_ml[k * NB * 32 + NB * 16 + cl] * f;
        v += part[u] * f;
      }
    }
    const float inv = 1.f / l;
    const int row = c % a.M, qh = h * a.group + c / a.M;
    float *dst = a.o + ((size_t)row * a.hq + qh) * HEAD_D + d * 16 + 4 * (ln >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[r] = v[r] * inv;
  }
  if (tid == 0) __hip_atomic_store(&a.cnt[hz], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Rows [n][Hkv][D] (bf16) -> cache positions pos0 .. pos0 + n - 1, fragment
// order. One thread per (row, head, 8 consecutive d).
__global__ void k_kv_write(const uint16_t *__restrict__ krows, const uint16_t *__restrict__ vrows, int n,
                           int64_t pos0, int hkv, int64_t cap, uint16_t *__restrict__ kc,
                           uint16_t *__restrict__ vc) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)n * hkv * (HEAD_D / 8);
  if (idx >= total) return;
  const int c8 = (int)(idx % (HEAD_D / 8));
  const int h = (int)((idx / (HEAD_D / 8)) % hkv);
  const int64_t r = idx / ((int64_t)(HEAD_D / 8) * hkv);
  const int64_t p = pos0 + r;
  const int d0 = 8 * c8;
  const size_t src = ((size_t)r * hkv + h) * HEAD_D + d0;
  // keys: 8 consecutive d are one lane's 16 bytes
  {
    const int s = d0 / 32, g = (d0 % 32) / 8;
    const int lane = g * 16 + (int)(p % 16);
    const size_t dst = ((((size_t)h * (size_t)(cap / 16) + (size_t)(p / 16)) * KSTEP + s) * 64 + lane) * 8;
    *reinterpret_cast<uint4 *>(kc + dst) = *reinterpret_cast<const uint4 *>(krows + src);
  }
  // values: position p is slot j of lane group g in its 32-group; each d is
  // another lane
  {
    const int q = (int)(p % 32), t = q / 16, rr = q % 16;
    const int g = rr / 4, j = (rr % 4) + 4 * t;
    const uint4 raw = *reinterpret_cast<const uint4 *>(vrows + src);
    uint16_t vals[8];
    __builtin_memcpy(vals, &raw, 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = d0 + e;
      const int lane = g * 16 + (d % 16);
      const size_t dst = ((((size_t)h * (size_t)(cap / 32) + (size_t)(p / 32)) * DBLK + d / 16) * 64 + lane) * 8 + j;
      vc[dst] = vals[e];
    }
  }
}

struct AttnPlan {
  int nb, ncb, nchunks, chunk;  // column blocks per work-group, work-groups per (head, chunk)
  size_t rec_floats;
};
// Arrival tickets at the start of the workspace: one per (head, work-group
// of column blocks).
constexpr size_t TICKET_BYTES = 1024;

constexpr int MAX_CHUNKS = 64;
// At least 352 positions a chunk (11 groups of 32, about three per wave):
// measured at 40 heads, 1k context, M = 16 / 32: 14.9 / 21.3 us with 3 chunks
// against 16.2 / 24.1 with 9 chunks of 128 and 20.4 / 31.2 with one.
constexpr int MIN_CHUNK_POS = 352;
// Contexts up to this many positions split two column blocks over two
// work-groups, one per CU (3 chunks a head at 40 heads): measured at 40 heads
// and M = 32, 21.2 / 26.2 / 36.3 / 52.7 us at 1k / 2k / 4k / 8k in one
// work-group, 14.8 / 20.5 / 31.1 / 50.7 split.
constexpr int64_t SPLIT_MAX_POS = 8192 + NVFP4V_ATTN_MAX_ROWS;

int attn_nb(int64_t m, int hq, int hkv) { return (int64_t)(hq / hkv) * m <= 16 ? 1 : 2; }

// Chunks per key/value head: one work-group per CU (chunks = CUs / Hkv), or,
// with two column blocks and chunks longer than 2048 positions, every
// work-group slot the kernel has (its work-groups per CU x CUs); at least 352
// positions a chunk, at most 64 chunks. Measured at 40 heads (µs, M = 16 / 32):
// one work-group per CU (6 chunks) against two (12 chunks) 25.5 / 35.2 vs
// 28.9 / 37.6 at 4k, 38.8 / 50.6 vs 43.6 / 53.3 at 8k, 68.7 / 83.8 vs
// 74.5 / 81.4 at 16k and 122.3 / 146.4 vs 131.7 / 137.8 at 32k. A wave of the
// one-block kernel keeps two groups of keys and values in flight, so one wave
// per SIMD streams at the full rate, and a head's last work-group then merges
// half as many records; the two-block kernel keeps one group in flight and
// needs the second work-group per CU once chunks are long.
void attn_plan(int64_t ctx_len, int64_t m, int hq, int hkv, int per_cu, int cus, AttnPlan *p) {
  p->nb = attn_nb(m, hq, hkv);
  p->ncb = 1;
  const int64_t P = ctx_len + m;
  int64_t nch = std::max<int64_t>(1, cus / hkv);
  // Two column blocks over a short context: one work-group per column block
  // (each reads the chunk's keys and values; the twin, 8-congruent in id, on
  // the same XCD), so that a wave keeps two groups in flight.
  const char *split_env = std::getenv("NVFP4V_ATTN_SPLIT");
  const bool split = p->nb == 2 && (split_env ? std::atoi(split_env) != 0 : P <= SPLIT_MAX_POS);
  if (split) {
    p->nb = 1;
    p->ncb = 2;
    nch = std::max<int64_t>(1, cus / (2 * hkv));
  } else if (p->nb == 2 && P > 2048 * nch) {
    nch = std::max<int64_t>(1, (int64_t)per_cu * cus / hkv);
  }
  nch = std::min<int64_t>({nch, (P + MIN_CHUNK_POS - 1) / MIN_CHUNK_POS, (int64_t)MAX_CHUNKS});
  // NVFP4V_ATTN_CHUNKS=<n> overrides the chunk count (for measurements; at
  // least one 32-position group per chunk, at most 64 chunks).
  if (const char *env = std::getenv("NVFP4V_ATTN_CHUNKS"))
    if (std::atoi(env) > 0)
      nch = std::min<int64_t>({(int64_t)std::atoi(env), (P + GROUP_POS - 1) / GROUP_POS, (int64_t)MAX_CHUNKS});
  nch = std::max<int64_t>(nch, 1);
  int64_t chunk = (P + nch - 1) / nch;
  chunk = (chunk + GROUP_POS - 1) / GROUP_POS * GROUP_POS;
  p->chunk = (int)chunk;
  p->nchunks = (int)((P + chunk - 1) / chunk);
  p->rec_floats = p->nb == 1 ? record_floats<1>() : record_floats<2>();
}

// The largest workspace any plan of the shape uses.
size_t attn_ws_bound(int64_t ctx_len, int64_t m, int hq, int hkv) {
  const int64_t P = ctx_len + m;
  const int64_t nch = std::min<int64_t>((P + MIN_CHUNK_POS - 1) / MIN_CHUNK_POS, MAX_CHUNKS);
  const size_t rec = attn_nb(m, hq, hkv) == 1 ? record_floats<1>() : record_floats<2>();
  return TICKET_BYTES + (size_t)hkv * (size_t)nch * rec * sizeof(float);
}

size_t attn_ws_bytes(const AttnPlan &p, int hkv) {
  return TICKET_BYTES + (size_t)hkv * p.ncb * p.nchunks * p.rec_floats * sizeof(float);
}

// Work-groups per CU the kernel of `nb` column blocks fits, and the CUs.
int attn_slots(nvfp4v_ctx *ctx, int nb, int *per_cu, int *cus) {
  int n = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &n, nb == 1 ? (const void *)k_tree_attn<1> : (const void *)k_tree_attn<2>, ATTN_THREADS, 0);
  if (e != hipSuccess) return hip_status(ctx, e);
  *per_cu = std::max(1, n);
  *cus = std::max(1, ctx->num_cus);
  return NVFP4V_OK;
}

int check_attn_shape(int64_t cap, int64_t ctx_len, int64_t m, int hq, int hkv, int d) {
  if (d != HEAD_D) return NVFP4V_E_SHAPE;
  if (hq < 1 || hkv < 1 || hq % hkv || hkv > 64) return NVFP4V_E_SHAPE;
  if (m < 1 || m > NVFP4V_ATTN_MAX_ROWS || (int64_t)(hq / hkv) * m > NVFP4V_ATTN_MAX_ROWS) return NVFP4V_E_M_RANGE;
  if (ctx_len < 0 || cap < 32 || cap % 32 || ctx_len + m > cap || cap > ((int64_t)1 << 30)) return NVFP4V_E_SHAPE;
  return NVFP4V_OK;
}

}  // namespace

extern "C" size_t nvfp4v_kv_cache_bytes(int64_t cap, int hkv, int d) {
  if (d != HEAD_D || hkv < 1 || cap < 32 || cap % 32) return 0;
  return (size_t)cap * hkv * HEAD_D * sizeof(uint16_t);
}

extern "C" int nvfp4v_kv_write(nvfp4v_ctx *ctx, const uint16_t *k_rows, const uint16_t *v_rows, int64_t n,
                               int64_t pos0, int hkv, int d, int64_t cap, uint16_t *k_cache, uint16_t *v_cache,
                               hipStream_t stream) {
  if (!ctx || !k_rows || !v_rows || !k_cache || !v_cache) return NVFP4V_E_INVALID_ARG;
  if (d != HEAD_D || hkv < 1 || hkv > 64 || cap < 32 || cap % 32 || cap > ((int64_t)1 << 30)) return NVFP4V_E_SHAPE;
  if (n < 1 || pos0 < 0 || pos0 + n > cap) return NVFP4V_E_SHAPE;
  if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(k_cache) || !aligned16(v_cache)) return NVFP4V_E_ALIGN;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const int64_t total = n * hkv * (HEAD_D / 8);
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return NVFP4V_E_SHAPE;
  hipLaunchKernelGGL(k_kv_write, dim3((unsigned)blocks), dim3(256), 0, stream, k_rows, v_rows, (int)n, pos0, hkv, cap,
                     k_cache, v_cache);
  return hip_status(ctx, hipGetLastError());
}

extern "C" size_t nvfp4v_tree_attention_workspace_bytes(int64_t ctx_len, int64_t m, int hq, int hkv, int d) {
  if (check_attn_shape(std::max<int64_t>(32, (ctx_len + m + 31) / 32 * 32), ctx_len, m, hq, hkv, d) != NVFP4V_OK)
    return 0;
  return attn_ws_bound(ctx_len, m, hq, hkv);
}

extern "C" int nvfp4v_tree_attention(nvfp4v_ctx *ctx, const uint16_t *q, const uint16_t *k_cache,
                                     const uint16_t *v_cache, int64_t cap, int64_t ctx_len, int64_t m, int hq,
                                     int hkv, int d, const int32_t *parent_rows, float scale, float *o, void *ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!ctx || !q || !k_cache || !v_cache || !parent_rows || !o || !ws) return NVFP4V_E_INVALID_ARG;
  int rc = check_attn_shape(cap, ctx_len, m, hq, hkv, d);
  if (rc) return rc;
  if (!std::isfinite(scale)) return NVFP4V_E_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) || !aligned16(ws))
    return NVFP4V_E_ALIGN;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  // Rows see themselves and their ancestors: parent_rows[0] = -1 (the root),
  // 0 <= parent_rows[i] < i otherwise.
  if (parent_rows[0] != -1) return NVFP4V_E_INVALID_ARG;
  a.vis[0] = 1u;
  for (int64_t i = 1; i < m; ++i) {
    const int32_t pr = parent_rows[i];
    if (pr < 0 || pr >= i) return NVFP4V_E_INVALID_ARG;
    a.vis[i] = a.vis[pr] | (1u << i);
  }
  int per_cu = 0, cus = 0;
  rc = attn_slots(ctx, attn_nb(m, hq, hkv), &per_cu, &cus);
  if (rc) return rc;
  AttnPlan p;
  attn_plan(ctx_len, m, hq, hkv, per_cu, cus, &p);
  if (ws_bytes < attn_ws_bytes(p, hkv)) return NVFP4V_E_WORKSPACE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.o = o;
  a.cnt = reinterpret_cast<unsigned *>(ws);
  a.rec = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + TICKET_BYTES);
  a.cap = cap;
  a.T = (int)ctx_len;
  a.M = (int)m;
  a.hq = hq;
  a.hkv = hkv;
  a.group = hq / hkv;
  a.P = (int)(ctx_len + m);
  a.chunk = p.chunk;
  a.nchunks = p.nchunks;
  a.ncb = p.ncb;
  a.scale = scale;
  const dim3 grid((unsigned)p.nchunks, (unsigned)hkv, (unsigned)p.ncb);
  if (p.nb == 1)
    hipLaunchKernelGGL(k_tree_attn<1>, grid, dim3(ATTN_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(k_tree_attn<2>, grid, dim3(ATTN_THREADS), 0, stream, a);
  return hip_status(ctx, hipGetLastError());
}

extern "C" int nvfp4v_tree_attention_plan(nvfp4v_ctx *ctx, int64_t ctx_len, int64_t m, int hq, int hkv, int d,
                                          int *nchunks, int *chunk) {
  if (!ctx || !nchunks || !chunk) return NVFP4V_E_INVALID_ARG;
  int rc = check_attn_shape(std::max<int64_t>(32, (ctx_len + m + 31) / 32 * 32), ctx_len, m, hq, hkv, d);
  if (rc) return rc;
  int per_cu = 0, cus = 0;
  rc = attn_slots(ctx, attn_nb(m, hq, hkv), &per_cu, &cus);
  if (rc) return rc;
  AttnPlan p;
  attn_plan(ctx_len, m, hq, hkv, per_cu, cus, &p);
  *nchunks = p.nchunks;
  *chunk = p.chunk;
  return NVFP4V_OK;
}
