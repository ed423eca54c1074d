// Context lifetime, status codes and shared host helpers of the C ABI.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <new>

#include "internal.h"

namespace nvfp4v {

int fault_injected() {
  const char *f = std::getenv("NVFP4V_FAULT");
  return (f && std::strcmp(f, "launch") == 0) ? 1 : 0;
}

int hip_status(nvfp4v_ctx *ctx, hipError_t e) {
  if (e == hipSuccess) return NVFP4V_OK;
  if (ctx) ctx->last_hip = (int)e;
  return NVFP4V_E_HIP;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace nvfp4v

using namespace nvfp4v;

// Split-K workspace: partial sums for up to 8 Mi floats (32 MiB) and 4096
// row-block counters. The tile table keeps ksplit * M * N_pad within it.
static constexpr size_t kPartialFloats = size_t(8) << 20;
static constexpr size_t kCounters = 4096;
// Packed-activation buffer of nvfp4v_verify_gemm: 16 MiB covers M = 64 up to
// K = 131072 (larger requests return NVFP4V_E_WORKSPACE).
static constexpr size_t kActBytes = size_t(16) << 20;

extern "C" int nvfp4v_create(nvfp4v_ctx **out, int device, const char *tile_table_path) {
  if (!out || device < 0) return NVFP4V_E_INVALID_ARG;
  *out = nullptr;
  if (fault_injected()) return NVFP4V_E_FAULT;
  nvfp4v_ctx *ctx = new (std::nothrow) nvfp4v_ctx();
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  if (tile_table_path) {
    const int rc = nvfp4v_load_tile_table(ctx, tile_table_path);
    if (rc) {
      delete ctx;
      return rc;
    }
  }
  ctx->device = device;
  hipError_t e = hipSetDevice(device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->partials, kPartialFloats * sizeof(float));
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->counters, kCounters * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(ctx->counters, 0, kCounters * sizeof(unsigned));
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->act, kActBytes);
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->pass_sync, PASS_SYNC_WORDS * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(ctx->pass_sync, 0, PASS_SYNC_WORDS * sizeof(unsigned));
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->dev_status, DEV_STATUS_BYTES);
  if (e == hipSuccess) e = hipMemset(ctx->dev_status, 0, DEV_STATUS_BYTES);
  const char *tl = std::getenv("NVFP4V_PASS_TRACE");
  if (e == hipSuccess && tl && std::strcmp(tl, "1") == 0) {
    ctx->pass_timeline_words = 2 * PASS_TIMELINE_WGS * PASS_TIMELINE_PHASES;
    e = hipMalloc((void **)&ctx->pass_timeline, ctx->pass_timeline_words * sizeof(uint64_t));
    if (e == hipSuccess) e = hipMemset(ctx->pass_timeline, 0, ctx->pass_timeline_words * sizeof(uint64_t));
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    int code = (int)e;
    nvfp4v_destroy(ctx);
    (void)code;
    return NVFP4V_E_HIP;
  }
  ctx->partial_floats = kPartialFloats;
  ctx->n_counters = kCounters;
  ctx->act_bytes = kActBytes;
  if (probe_dispatch(ctx) != NVFP4V_OK) {
    nvfp4v_destroy(ctx);
    return NVFP4V_E_HIP;
  }
  *out = ctx;
  return NVFP4V_OK;
}

extern "C" void nvfp4v_destroy(nvfp4v_ctx *ctx) {
  if (!ctx) return;
  if (ctx->partials) (void)hipFree(ctx->partials);
  if (ctx->counters) (void)hipFree(ctx->counters);
  if (ctx->act) (void)hipFree(ctx->act);
  if (ctx->pass_sync) (void)hipFree(ctx->pass_sync);
  if (ctx->pass_timeline) (void)hipFree(ctx->pass_timeline);
  if (ctx->dev_status) (void)hipFree(ctx->dev_status);
  delete ctx;
}

extern "C" int nvfp4v_device_status(nvfp4v_ctx *ctx) {
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  unsigned w[DEV_STATUS_BYTES / sizeof(unsigned)];
  if (e == hipSuccess) e = hipMemcpy(w, ctx->dev_status, DEV_STATUS_BYTES, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(ctx, e);
  unsigned begun = 0, done = 0;  // modulo 2^32 on both sides
  for (int x = 0; x < 8; ++x) {
    begun += w[x * DEV_LINE_WORDS + DEV_ROWS_BEGUN];
    done += w[x * DEV_LINE_WORDS + DEV_ROWS_DONE];
  }
  if (begun == done) return NVFP4V_OK;
  // Some row block's pieces ran on two XCDs, so their tickets went to two
  // L2s and its C was never written. Clear the counts and the tickets, and
  // exchange through memory from now on.
  ctx->xcd_local = 0;
  e = hipMemset(ctx->dev_status, 0, DEV_STATUS_BYTES);
  if (e == hipSuccess) e = hipMemset(ctx->counters, 0, ctx->n_counters * sizeof(unsigned));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_status(ctx, e);
  return NVFP4V_E_DISPATCH;
}

extern "C" int nvfp4v_f16_redone(nvfp4v_ctx *ctx, uint64_t *units) {
  if (!ctx || !units) return NVFP4V_E_INVALID_ARG;
  hipError_t e = hipSetDevice(ctx->device);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  unsigned w[DEV_STATUS_BYTES / sizeof(unsigned)];
  if (e == hipSuccess) e = hipMemcpy(w, ctx->dev_status, DEV_STATUS_BYTES, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(ctx, e);
  uint64_t n = 0;
  for (int x = 0; x < 8; ++x) n += w[x * DEV_LINE_WORDS + DEV_F16_REDONE];
  *units = n;
  return NVFP4V_OK;
}

extern "C" size_t nvfp4v_ctx_size(void) { return sizeof(nvfp4v_ctx); }

extern "C" int nvfp4v_last_hip_error(const nvfp4v_ctx *ctx) { return ctx ? ctx->last_hip : 0; }

extern "C" int nvfp4v_set_pass_mode(nvfp4v_ctx *ctx, int mode) {
  if (!ctx || (mode != NVFP4V_PASS_CHAIN && mode != NVFP4V_PASS_PERSISTENT))
    return NVFP4V_E_INVALID_ARG;
  ctx->pass_mode = mode;
  return NVFP4V_OK;
}

extern "C" int nvfp4v_get_pass_mode(const nvfp4v_ctx *ctx) { return ctx ? ctx->pass_mode : NVFP4V_E_INVALID_ARG; }

extern "C" int nvfp4v_last_pass_grid(const nvfp4v_ctx *ctx) { return ctx ? ctx->last_pass_grid : 0; }

extern "C" int nvfp4v_pass_timeline(nvfp4v_ctx *ctx, uint64_t *out, size_t max_words, int *phases,
                                    int *groups) {
  if (!ctx || !out || !phases || !groups) return NVFP4V_E_INVALID_ARG;
  if (!ctx->pass_timeline) return NVFP4V_E_INVALID_ARG;
  const size_t n = std::min(max_words, ctx->pass_timeline_words);
  hipError_t e = hipMemcpy(out, ctx->pass_timeline, n * sizeof(uint64_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_status(ctx, e);
  *phases = ctx->last_pass_phases;
  *groups = ctx->last_pass_grid;
  return NVFP4V_OK;
}

extern "C" const char *nvfp4v_strerror(int status) {
  switch (status) {
    case NVFP4V_OK: return "ok";
    case NVFP4V_E_INVALID_ARG: return "invalid argument (null pointer or context)";
    case NVFP4V_E_SHAPE: return "bad shape (need N >= 1, K >= 16, K % 16 == 0)";
    case NVFP4V_E_M_RANGE: return "M out of range";
    case NVFP4V_E_ALIGN: return "device pointer not 16-byte aligned";
    case NVFP4V_E_HIP: return "HIP runtime or launch error";
    case NVFP4V_E_FAULT: return "injected fault (NVFP4V_FAULT=launch)";
    case NVFP4V_E_NONFINITE: return "non-finite input";
    case NVFP4V_E_WORKSPACE: return "request exceeds the context's split-K workspace";
    case NVFP4V_E_TIMEOUT: return "a persistent pass timed out at a grid barrier";
    case NVFP4V_E_DISPATCH: return "the pieces of a split-K row block ran on different XCDs (outputs undefined)";
    case NVFP4V_E_TABLE: return "tile table unreadable or malformed (or for another arch)";
    default: return "unknown status";
  }
}
