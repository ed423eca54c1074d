// Context lifetime, status codes and shared host helpers of the C ABI.
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

extern "C" int nvfp4v_create(nvfp4v_ctx **out, int device) {
  if (!out || device < 0) return NVFP4V_E_INVALID_ARG;
  *out = nullptr;
  if (fault_injected()) return NVFP4V_E_FAULT;
  nvfp4v_ctx *ctx = new (std::nothrow) nvfp4v_ctx();
  if (!ctx) return NVFP4V_E_INVALID_ARG;
  ctx->device = device;
  hipError_t e = hipSetDevice(device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ctx->num_cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->partials, kPartialFloats * sizeof(float));
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->counters, kCounters * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(ctx->counters, 0, kCounters * sizeof(unsigned));
  if (e == hipSuccess) e = hipMalloc((void **)&ctx->act, kActBytes);
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
  *out = ctx;
  return NVFP4V_OK;
}

extern "C" void nvfp4v_destroy(nvfp4v_ctx *ctx) {
  if (!ctx) return;
  if (ctx->partials) (void)hipFree(ctx->partials);
  if (ctx->counters) (void)hipFree(ctx->counters);
  if (ctx->act) (void)hipFree(ctx->act);
  delete ctx;
}

extern "C" int nvfp4v_last_hip_error(const nvfp4v_ctx *ctx) { return ctx ? ctx->last_hip : 0; }

extern "C" const char *nvfp4v_strerror(int status) {
  switch (status) {
    case NVFP4V_OK: return "ok";
    case NVFP4V_E_INVALID_ARG: return "invalid argument (null pointer or context)";
    case NVFP4V_E_SHAPE: return "bad shape (need N >= 1, K >= 16, K % 16 == 0)";
    case NVFP4V_E_M_RANGE: return "M out of range (1..64)";
    case NVFP4V_E_ALIGN: return "device pointer not 16-byte aligned";
    case NVFP4V_E_HIP: return "HIP runtime or launch error";
    case NVFP4V_E_FAULT: return "injected fault (NVFP4V_FAULT=launch)";
    case NVFP4V_E_NONFINITE: return "non-finite input";
    case NVFP4V_E_WORKSPACE: return "request exceeds the context's split-K workspace";
    default: return "unknown status";
  }
}
