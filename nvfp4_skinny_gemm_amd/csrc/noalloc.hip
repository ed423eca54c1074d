// nvfp4v_verify_gemm_static: the verify GEMM for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). It needs no context: the scratch memory the GEMM's kernels use
// (the packed activations, the split-K partial sums and the arrival counters)
// is one file-scope device array, `scratch`, of SCRATCH_BYTES, which every GPU
// the library runs on holds until the process ends. Host code never passes the
// array's name to a kernel (in host code it is a stand-in, not a device
// address): the first call on a device looks up that device's copy with
// hipGetSymbolAddress and keeps the address; every later use goes through it.
//
// The plan is the built-in tile table's, with the split-K partials exchanged
// through memory (no dispatch probe runs here), which sums in the same order
// as the context's exchange, so C equals nvfp4v_verify_gemm's bitwise.
#include <algorithm>
#include <mutex>

#include "internal.h"

using namespace nvfp4v;

namespace {

constexpr size_t COUNTER_WORDS = 4096;
constexpr size_t COUNTER_BYTES = COUNTER_WORDS * sizeof(unsigned);  // 16 KiB
constexpr size_t ACT_OFFSET = 64 << 10;
constexpr size_t ACT_CAP = size_t(16) << 20;      // packed activations of one 64-row block (both copies)
constexpr size_t PART_OFFSET = ACT_OFFSET + ACT_CAP;
constexpr size_t PART_CAP = size_t(8) << 20;      // split-K partial sums
constexpr size_t SCRATCH_BYTES = PART_OFFSET + PART_CAP;

__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
uint8_t *g_scratch[MAX_DEVICES] = {};

// This device's copy of the array (looked up once per device).
hipError_t scratch_address(int device, uint8_t **out) {
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[device]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[device] = static_cast<uint8_t *>(p);
  }
  *out = g_scratch[device];
  return hipSuccess;
}

__global__ void k_clear_counters(unsigned *w, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) w[i] = 0u;
}

}  // namespace

extern "C" int nvfp4v_verify_gemm_static(const uint16_t *a, int64_t m, int64_t k, const void *packed, int64_t n,
                                         float ts, float *c, hipStream_t stream) {
  if (!a || !packed || !c) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  Layout L;
  if (!make_layout(n, k, &L)) return NVFP4V_E_SHAPE;
  if (!aligned16(a) || !aligned16(packed) || !aligned16(c)) return NVFP4V_E_ALIGN;
  if (2 * act_block_bytes(std::min<int64_t>(m, CHUNK_M), k) > ACT_CAP) return NVFP4V_E_WORKSPACE;
  // A context on the stack (no allocation) whose workspace is the scratch
  // array: built-in tile table, exchange through memory.
  nvfp4v_ctx local;
  for (int64_t r0 = 0; r0 < m; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    Plan p;
    const int rc = make_plan(&local, L, mc, &p);
    if (rc) return rc;
    if (p.ksplit > 1 && ((size_t)p.ksplit * (size_t)mc * (size_t)(L.nrt * ROWS_PER_TILE) > PART_CAP / sizeof(float) ||
                         (size_t)p.nrb > COUNTER_WORDS))
      return NVFP4V_E_WORKSPACE;
  }
  if (fault_injected()) return NVFP4V_E_FAULT;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return NVFP4V_E_HIP;
  if (device < 0 || device >= MAX_DEVICES) return NVFP4V_E_INVALID_ARG;
  uint8_t *base = nullptr;
  e = scratch_address(device, &base);
  if (e != hipSuccess) return NVFP4V_E_HIP;
  local.device = device;
  local.counters = reinterpret_cast<unsigned *>(base);
  local.n_counters = COUNTER_WORDS;
  local.act = base + ACT_OFFSET;
  local.act_bytes = ACT_CAP;
  local.partials = reinterpret_cast<float *>(base + PART_OFFSET);
  local.partial_floats = PART_CAP / sizeof(float);
  local.xcd_local = 0;
  // The arrival counters start every call at zero (a kernel, not a memset, so
  // the call can be captured in a graph).
  hipLaunchKernelGGL(k_clear_counters, dim3(16), dim3(256), 0, stream, local.counters, (int)COUNTER_WORDS);
  int rc = hip_status(&local, hipGetLastError());
  const bool f16 = use_f16();
  for (int64_t r0 = 0; r0 < m && rc == NVFP4V_OK; r0 += CHUNK_M) {
    const int64_t mc = std::min<int64_t>(CHUNK_M, m - r0);
    const size_t act16 = act_block_bytes(mc, k);
    rc = launch_pack_act(&local, a + r0 * k, mc, k, local.act, act16, stream);
    if (!rc) rc = launch_gemm(&local, local.act, f16 ? act16 : 0, mc, k, packed, n, ts, c + r0 * n, stream);
  }
  return rc;
}
