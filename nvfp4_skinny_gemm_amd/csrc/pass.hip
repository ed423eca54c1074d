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
#include <hip/hip_bf16.h>

#include <cmath>

#include "internal.h"

using namespace nvfp4v;

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

// Fused chain glue for the pass: each thread turns 8 consecutive outputs of a
// row into bf16 and writes them as one 16-byte chunk of the next GEMM's packed
// activations (and, when asked, into up to two row-major bf16 copies).
// y == nullptr: out = bf16(x * c); otherwise out = bf16(x * c + y * c).
__global__ void k_glue_pa(const float *__restrict__ x, int64_t ldx, const float *__restrict__ y,
                          int64_t ldy, int rows, int cols, float c, uint8_t *__restrict__ act,
                          int mblocks, uint16_t *__restrict__ rm0, uint16_t *__restrict__ rm1) {
#pragma clang fp contract(off)
  const int chunks = cols / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * chunks) return;
  const int r = (int)(idx / chunks), k0 = (int)(idx - (int64_t)r * chunks) * 8;
  uint16_t o[8];
  const float *xr = x + (size_t)r * ldx + k0;
  if (y) {
    const float *yr = y + (size_t)r * ldy + k0;
    for (int e = 0; e < 8; ++e) {
      const float px = xr[e] * c;
      const float py = yr[e] * c;
      o[e] = to_bf16_bits(px + py);
    }
  } else {
    for (int e = 0; e < 8; ++e) o[e] = to_bf16_bits(xr[e] * c);
  }
  uint4 v;
  __builtin_memcpy(&v, o, 16);
  *reinterpret_cast<uint4 *>(act + act_offset(r, k0, mblocks)) = v;
  if (rm0) *reinterpret_cast<uint4 *>(rm0 + (size_t)r * cols + k0) = v;
  if (rm1) *reinterpret_cast<uint4 *>(rm1 + (size_t)r * cols + k0) = v;
}

int launch_glue_pa(nvfp4v_ctx *ctx, const float *x, int64_t ldx, const float *y, int64_t ldy,
                   int64_t rows, int64_t cols, float c, uint8_t *act, uint16_t *rm0, uint16_t *rm1,
                   hipStream_t stream) {
  const int64_t total = rows * (cols / 8);
  const int mblocks = (int)((rows + 15) / 16);
  hipLaunchKernelGGL(k_glue_pa, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, x, ldx,
                     y, ldy, (int)rows, (int)cols, c, act, mblocks, rm0, rm1);
  return hip_status(ctx, hipGetLastError());
}

unsigned glue_grid(int64_t total) {
  const int64_t g = (total + 255) / 256;
  return (unsigned)(g < 2048 ? (g > 0 ? g : 1) : 2048);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct PassWs {
  float *qkv, *o, *gu, *d;
  uint8_t *act_h, *act_o, *act_g, *act_d;  // packed activations of the four GEMMs
};

size_t pass_ws_layout(int64_t m, int64_t H, int64_t I, uint8_t *base, PassWs *w) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    uint8_t *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w->qkv = (float *)take((size_t)m * 3 * H * 4);
  w->o = (float *)take((size_t)m * H * 4);
  w->gu = (float *)take((size_t)m * 2 * I * 4);
  w->d = (float *)take((size_t)m * H * 4);
  w->act_h = take(act_packed_bytes(m, H));
  w->act_o = take(act_packed_bytes(m, H));
  w->act_g = take(act_packed_bytes(m, H));
  w->act_d = take(act_packed_bytes(m, I));
  return off;
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

extern "C" size_t nvfp4v_pass_workspace_bytes(int64_t m, int64_t hidden, int64_t inter) {
  if (m < 1 || m > NVFP4V_MAX_M || hidden < 16 || inter < 16) return 0;
  PassWs w;
  return pass_ws_layout(m, hidden, inter, nullptr, &w);
}

extern "C" int nvfp4v_verify_pass(nvfp4v_ctx *ctx, const nvfp4v_layer *layers, int n_layers,
                                  int64_t hidden, int64_t inter, const uint16_t *h0, int64_t m,
                                  void *ws, size_t ws_bytes, uint16_t *h_out, uint16_t *trace,
                                  hipStream_t stream) {
  if (!ctx || !layers || !h0 || !ws || !h_out) return NVFP4V_E_INVALID_ARG;
  if (n_layers < 1) return NVFP4V_E_INVALID_ARG;
  if (m < 1 || m > NVFP4V_MAX_M) return NVFP4V_E_M_RANGE;
  if (hidden < 16 || inter < 16 || hidden % 16 || inter % 16) return NVFP4V_E_SHAPE;
  if (!aligned16(h0) || !aligned16(ws) || !aligned16(h_out) || (trace && !aligned16(trace)))
    return NVFP4V_E_ALIGN;
  for (int l = 0; l < n_layers; ++l)
    if (!layers[l].qkv || !layers[l].o || !layers[l].gate_up || !layers[l].down)
      return NVFP4V_E_INVALID_ARG;
  PassWs w;
  const size_t need = pass_ws_layout(m, hidden, inter, (uint8_t *)ws, &w);
  if (ws_bytes < need) return NVFP4V_E_WORKSPACE;
  if (fault_injected()) return NVFP4V_E_FAULT;
  const float ch = (float)(1.0 / std::sqrt((double)hidden));
  const float ci = (float)(1.0 / std::sqrt((double)inter));
  const float c2h = (float)(1.0 / std::sqrt(2.0 * (double)hidden));
  const int64_t H = hidden, I = inter;
  int rc = launch_pack_act(ctx, h0, m, H, w.act_h, stream);
  // Each GEMM's epilogue writes the next GEMM's packed activations (the glue
  // above), so a layer is four launches.
  Epilogue e_o, e_g, e_d, e_h;
  e_o.mode = EPI_SCALE, e_o.col0 = (int)(2 * H), e_o.col1 = (int)(3 * H), e_o.c = ch, e_o.act = w.act_o;
  e_g.mode = EPI_SCALE, e_g.col0 = 0, e_g.col1 = (int)H, e_g.c = ch, e_g.act = w.act_g;
  e_d.mode = EPI_PAIR, e_d.c = c2h, e_d.act = w.act_d;
  e_h.mode = EPI_SCALE, e_h.col0 = 0, e_h.col1 = (int)H, e_h.c = ci, e_h.act = w.act_h;
  for (int l = 0; l < n_layers && rc == NVFP4V_OK; ++l) {
    const nvfp4v_layer &L = layers[l];
    e_h.rm0 = (l == n_layers - 1) ? h_out : nullptr;
    e_h.rm1 = trace ? trace + (size_t)l * m * H : nullptr;
    rc = launch_gemm(ctx, w.act_h, m, H, L.qkv, 3 * H, L.ts_qkv, w.qkv, stream, e_o);
    if (!rc) rc = launch_gemm(ctx, w.act_o, m, H, L.o, H, L.ts_o, w.o, stream, e_g);
    if (!rc) rc = launch_gemm(ctx, w.act_g, m, H, L.gate_up, 2 * I, L.ts_gate_up, w.gu, stream, e_d);
    if (!rc) rc = launch_gemm(ctx, w.act_d, m, I, L.down, H, L.ts_down, w.d, stream, e_h);
  }
  return rc;
}
