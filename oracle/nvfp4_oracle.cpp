// NVFP4 verify-GEMM oracle: plain, slow, obviously correct CPU reference.
//
// TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
// this file; only the test suite, the smoke check and the CPU-baseline leg of
// the benchmark do. It shares no source, header, table or helper with the HIP
// library.
//
// What it computes (the plain definition; the GPU path must reach the same
// result up to fp32 rounding of its sums):
//   w(j,k)  = E2M1(code(j,k)) * E4M3(scale(j, k/16)) * ts           exact in fp64
//   C[i][j] = sum_{k ascending} a(i,k) * w(j,k)                      fp64
//   S[i][j] = sum_k |a(i,k) * w(j,k)|                                fp64
// Sources, by page:
//   * TandemLLM manual, "What TandemLLM is", 1.2 "Two levers": every projection
//     is stored with four bits per weight and one scale per 16 weights; a
//     verify pass applies those weights to all rows of the draft tree at once.
//   * Same page, 1.7 "The paper": the 4-bit kernels keep a fixed reduction
//     order (here: k ascending, one fp64 accumulator).
//   * Research page (StairCut), "What it says": the check is one pass over up
//     to 32 tree rows.
// The pages do not give the bit layout. The plainest reading that the rest
// supports, used here: each 4-bit code is an OCP E2M1 value (sign, 2 exponent
// bits with bias 1, 1 mantissa bit), each scale is an OCP E4M3 ("FN", bias 7,
// no infinities, 0x7F/0xFF are NaN) byte covering 16 consecutive elements along
// the reduction axis K, the low nibble of a code byte holds the even k, and an
// fp32 tensor scale multiplies every weight.
//
// Precision: every decode is exact in fp64 (8 + 2 + 4 + 24 = 38 significant
// bits <= 53). The chain glue is the only fp32 arithmetic here, because its
// result decides a bf16 bit pattern and both sides must take that decision in
// the same (fp32) precision.
//
// Parity pins (checked by the CPU test suite, not by this file): exhaustive
// E2M1 / E4M3 decode against closed forms and a library fp8 routine, a
// hand-computed 2x16x2 worked example, row independence, linearity, one-hot
// extraction, scale-exponent doubling, brute-force quantiser argmin, and a
// dense fp64 matmul of the decoded weights.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <sched.h>

namespace {

// ---- E2M1: 4-bit code s e1 e0 m --------------------------------------------
// Value (-1)^s * (e == 0 ? m/2 : 2^(e-1) * (1 + m/2)); magnitudes
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Code 8 is negative zero.
double e2m1_value(unsigned code) {
  code &= 0xFu;
  const unsigned s = (code >> 3) & 1u;
  const unsigned e = (code >> 1) & 3u;
  const unsigned m = code & 1u;
  double mag;
  if (e == 0)
    mag = 0.5 * (double)m;
  else
    mag = std::ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

// ---- E4M3 (OCP "FN"): byte s eeee mmm, bias 7 -------------------------------
// e == 0: subnormal (-1)^s * 2^-6 * m/8; e == 15 && m == 7: NaN; otherwise
// (-1)^s * 2^(e-7) * (1 + m/8). Largest finite magnitude 448.
double e4m3_value(unsigned byte) {
  byte &= 0xFFu;
  const unsigned s = (byte >> 7) & 1u;
  const unsigned e = (byte >> 3) & 15u;
  const unsigned m = byte & 7u;
  if (e == 15 && m == 7) return std::nan("");
  double mag;
  if (e == 0)
    mag = std::ldexp((double)m / 8.0, -6);
  else
    mag = std::ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

// Round-to-nearest, ties-to-even, onto the finite E4M3 grid, saturating at
// +-448. Works on the magnitude and keeps the sign. Input must not be NaN.
uint8_t e4m3_encode(double x) {
  const bool neg = std::signbit(x);
  double ax = std::fabs(x);
  uint8_t mag;
  if (ax >= 448.0) {
    mag = 0x7E;  // saturate (464 and above would otherwise round past 448)
  } else if (ax < std::ldexp(1.0, -6)) {
    // subnormal binade: grid step 2^-9; q = 8 means 2^-6, which is the
    // smallest normal and has the same bit pattern (e = 1, m = 0).
    const double q = std::nearbyint(ax / std::ldexp(1.0, -9));
    mag = (uint8_t)q;
  } else {
    int ex;
    (void)std::frexp(ax, &ex);  // ax = f * 2^ex, f in [0.5, 1)
    const int E = ex - 1;       // ax in [2^E, 2^(E+1))
    double q = std::nearbyint(ax / std::ldexp(1.0, E - 3));  // in [8, 16]
    int Eb = E;
    if (q >= 16.0) {
      q = 8.0;
      Eb = E + 1;
    }
    const int efield = Eb + 7;
    const int mfield = (int)q - 8;
    if (efield > 15 || (efield == 15 && mfield > 6))
      mag = 0x7E;  // cannot happen below 448, kept as a guard
    else
      mag = (uint8_t)((efield << 3) | mfield);
  }
  return (uint8_t)(mag | (neg ? 0x80 : 0x00));
}

// Round-to-nearest onto the E2M1 magnitudes, ties to the even mantissa bit,
// saturating at 6. The sign of q is kept, so -0 and tiny negatives give code 8.
uint8_t e2m1_encode(double q) {
  const bool neg = std::signbit(q);
  const double aq = std::fabs(q);
  int best = 0;
  double bestd = INFINITY;
  for (int c = 0; c < 8; ++c) {
    const double d = std::fabs(aq - e2m1_value((unsigned)c));
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
      bestd = d;
      best = c;
    }
  }
  if (aq > 6.0) best = 7;  // saturate
  return (uint8_t)(best | (neg ? 8 : 0));
}

inline double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

inline uint16_t bf16_from_float_rne(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);  // quiet NaN, sign kept
  const uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

int thread_count(int requested) {
  if (requested > 0) return requested;
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  unsigned h = std::thread::hardware_concurrency();
  return h ? (int)h : 1;
}

template <class F>
void parallel_rows(int64_t count, int threads, F fn) {
  threads = thread_count(threads);
  if (threads > count) threads = (int)(count > 0 ? count : 1);
  if (threads <= 1) {
    for (int64_t j = 0; j < count; ++j) fn(j);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t) {
    pool.emplace_back([=]() {
      for (int64_t j = t; j < count; j += threads) fn(j);
    });
  }
  for (auto &th : pool) th.join();
}

// Decode one weight row j of the canonical format into w[0..k).
void decode_row(const uint8_t *codes, const uint8_t *scales, int64_t k, int64_t j,
                double ts, double *w) {
  const uint8_t *crow = codes + j * (k / 2);
  const uint8_t *srow = scales + j * (k / 16);
  for (int64_t kk = 0; kk < k; ++kk) {
    const uint8_t byte = crow[kk >> 1];
    const unsigned code = (kk & 1) ? (byte >> 4) : (byte & 0xF);
    w[kk] = e2m1_value(code) * e4m3_value(srow[kk / 16]) * ts;
  }
}

}  // namespace

extern "C" {

int oracle_thread_count(void) { return thread_count(0); }

double oracle_e2m1_value(int code) { return e2m1_value((unsigned)code); }
double oracle_e4m3_value(int byte) { return e4m3_value((unsigned)byte); }

// Returns 0, or -1 for a NaN input.
int oracle_e4m3_encode(double x, uint8_t *out) {
  if (std::isnan(x)) return -1;
  *out = e4m3_encode(x);
  return 0;
}

int oracle_e2m1_encode(double q, uint8_t *out) {
  if (std::isnan(q)) return -1;
  *out = e2m1_encode(q);
  return 0;
}

// Quantise fp32 weights w[n][k] (k % 16 == 0) to the canonical format:
//   codes[n][k/2] (low nibble = even k), scales[n][k/16] E4M3.
// Per 16-element block along k: s = E4M3_RNE(absmax / 6) (fp64, saturating at
// 448); if s == 0 every code is +0; otherwise code = E2M1_RNE(w / s) (fp64,
// saturating at 6, sign kept). Non-finite input returns -1 and leaves the
// outputs unspecified. The scale rule (block absmax over the largest code
// magnitude, 6) is the standard NVFP4 recipe; the pages only say the weights
// were quantised onto the NVFP4 grid ("Installing TandemLLM", 3.12).
int oracle_quantize(const float *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales,
                    int threads) {
  if (k % 16 != 0 || n < 0 || k < 0) return -2;
  for (int64_t i = 0; i < n * k; ++i)
    if (!std::isfinite(w[i])) return -1;
  parallel_rows(n, threads, [&](int64_t j) {
    const float *wr = w + j * k;
    uint8_t *cr = codes + j * (k / 2);
    uint8_t *sr = scales + j * (k / 16);
    std::memset(cr, 0, (size_t)(k / 2));
    for (int64_t b = 0; b < k / 16; ++b) {
      double amax = 0.0;
      for (int t = 0; t < 16; ++t) amax = std::fmax(amax, std::fabs((double)wr[b * 16 + t]));
      const uint8_t sb = e4m3_encode(amax / 6.0);
      sr[b] = sb;
      const double s = e4m3_value(sb);
      for (int t = 0; t < 16; ++t) {
        const int64_t kk = b * 16 + t;
        const uint8_t c = (s == 0.0) ? 0 : e2m1_encode((double)wr[kk] / s);
        cr[kk >> 1] |= (uint8_t)((kk & 1) ? (c << 4) : c);
      }
    }
  });
  return 0;
}

// Decode the canonical format to dense fp64 w[n][k] (times ts).
void oracle_decode(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, double ts,
                   double *w) {
  for (int64_t j = 0; j < n; ++j) decode_row(codes, scales, k, j, ts, w + j * k);
}

// C[i][c] and S[i][c] for the weight rows listed in cols[0..ncols) (each a
// row index of the n x k weight matrix). a is m x k bf16 bit patterns,
// row-major. Outputs are m x ncols, row-major. Threaded over the listed rows;
// each output is one fp64 sum with k ascending.
void oracle_gemm_cols(const uint16_t *a, int64_t m, int64_t k, const uint8_t *codes,
                      const uint8_t *scales, const int64_t *cols, int64_t ncols, double ts,
                      double *c, double *s, int threads) {
  std::vector<double> av((size_t)(m * k));
  for (int64_t i = 0; i < m * k; ++i) av[(size_t)i] = bf16_value(a[i]);
  parallel_rows(ncols, threads, [&](int64_t idx) {
    std::vector<double> w((size_t)k);
    decode_row(codes, scales, k, cols[idx], ts, w.data());
    for (int64_t i = 0; i < m; ++i) {
      const double *ar = av.data() + i * k;
      double acc = 0.0, sacc = 0.0;
      for (int64_t kk = 0; kk < k; ++kk) {
        const double p = ar[kk] * w[(size_t)kk];
        acc += p;
        sacc += std::fabs(p);
      }
      c[i * ncols + idx] = acc;
      if (s) s[i * ncols + idx] = sacc;
    }
  });
}

// Full C = A * W^T for all n weight rows (codes/scales hold only those rows).
void oracle_gemm(const uint16_t *a, int64_t m, int64_t k, const uint8_t *codes,
                 const uint8_t *scales, int64_t n, double ts, double *c, double *s,
                 int threads) {
  std::vector<int64_t> cols((size_t)n);
  for (int64_t j = 0; j < n; ++j) cols[(size_t)j] = j;
  oracle_gemm_cols(a, m, k, codes, scales, cols.data(), n, ts, c, s, threads);
}

// ---- FP8 output head --------------------------------------------------------
// The served model keeps its output head in FP8 (TandemLLM manual, "What
// TandemLLM is", 1.2 "Two levers"; "Installing TandemLLM", 3.11 passes it as a
// separate checkpoint). The pages give neither the FP8 variant nor the scale
// granularity. The plainest reading, used here: OCP E4M3 codes (the same "FN"
// format as the NVFP4 block scales) with one fp32 scale per output row:
//   s(j)     = fp32( absmax_k |w(j,k)| / 448 )     (fp64 division, one rounding)
//   code     = E4M3_RNE( w(j,k) / s(j) )  (fp64, saturating at 448, sign kept);
//              every code is +0 when s(j) == 0
//   w8(j,k)  = s(j) * E4M3(code(j,k))              exact in fp64
//   C[i][j]  = sum_{k ascending} a(i,k) * w8(j,k)  fp64; S = sum of |terms|

// Quantise fp32 w[n][k] to E4M3 codes[n][k] and fp32 row scales[n]. Returns 0,
// -1 for a non-finite input, -2 for a bad shape.
int oracle_fp8_quantize(const float *w, int64_t n, int64_t k, uint8_t *codes, float *row_scales,
                        int threads) {
  if (n < 0 || k < 0) return -2;
  for (int64_t i = 0; i < n * k; ++i)
    if (!std::isfinite(w[i])) return -1;
  parallel_rows(n, threads, [&](int64_t j) {
    const float *wr = w + j * k;
    double amax = 0.0;
    for (int64_t kk = 0; kk < k; ++kk) amax = std::fmax(amax, std::fabs((double)wr[kk]));
    const float s = (float)(amax / 448.0);
    row_scales[j] = s;
    for (int64_t kk = 0; kk < k; ++kk)
      codes[j * k + kk] = (s == 0.0f) ? 0 : e4m3_encode((double)wr[kk] / (double)s);
  });
  return 0;
}

// C[i][c], S[i][c] (m x ncols, row-major) for the weight rows cols[0..ncols)
// of the FP8 head: codes[n][k], row_scales[n]; a is m x k bf16, row-major.
void oracle_fp8_gemm_cols(const uint16_t *a, int64_t m, int64_t k, const uint8_t *codes,
                          const float *row_scales, const int64_t *cols, int64_t ncols,
                          double *c, double *s, int threads) {
  std::vector<double> av((size_t)(m * k));
  for (int64_t i = 0; i < m * k; ++i) av[(size_t)i] = bf16_value(a[i]);
  parallel_rows(ncols, threads, [&](int64_t idx) {
    const int64_t j = cols[idx];
    const double sj = (double)row_scales[j];
    std::vector<double> w((size_t)k);
    for (int64_t kk = 0; kk < k; ++kk) w[(size_t)kk] = sj * e4m3_value(codes[j * k + kk]);
    for (int64_t i = 0; i < m; ++i) {
      const double *ar = av.data() + i * k;
      double acc = 0.0, sacc = 0.0;
      for (int64_t kk = 0; kk < k; ++kk) {
        const double p = ar[kk] * w[(size_t)kk];
        acc += p;
        sacc += std::fabs(p);
      }
      c[i * ncols + idx] = acc;
      if (s) s[i * ncols + idx] = sacc;
    }
  });
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
void oracle_bf16_from_f32(const float *x, int64_t count, uint16_t *out) {
  for (int64_t i = 0; i < count; ++i) out[i] = bf16_from_float_rne(x[i]);
}

// Chain glue between the GEMMs of one layer (elementwise, fp32, no fused ops):
//   out = bf16( x * c )                      (one fp32 product, then RNE)
void oracle_glue_scale(const float *x, int64_t count, float cst, uint16_t *out) {
  for (int64_t i = 0; i < count; ++i) {
    volatile float p = x[i] * cst;
    out[i] = bf16_from_float_rne(p);
  }
}

//   out = bf16( x * c + y * c )              (two fp32 products and one fp32
//                                             sum, no fused multiply-add, then RNE)
void oracle_glue_sum(const float *x, const float *y, int64_t count, float cst, uint16_t *out) {
  for (int64_t i = 0; i < count; ++i) {
    volatile float px = x[i] * cst;
    volatile float py = y[i] * cst;
    volatile float p = px + py;
    out[i] = bf16_from_float_rne(p);
  }
}

}  // extern "C"
