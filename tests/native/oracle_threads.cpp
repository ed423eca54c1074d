// Sanitizer driver for the oracle (test infrastructure): runs its threaded
// entry points (quantisers and GEMMs, NVFP4 and FP8) on seeded inputs with one
// and with several threads and checks that the results are bitwise equal.
// Built and run by tests/test_sanitizers.py under ThreadSanitizer and under
// AddressSanitizer + UndefinedBehaviorSanitizer; exits non-zero on a mismatch
// (a sanitizer report aborts the run by itself).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
int oracle_quantize(const float *w, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales, int threads);
void oracle_gemm(const uint16_t *a, int64_t m, int64_t k, const uint8_t *codes, const uint8_t *scales,
                 int64_t n, double ts, double *c, double *s, int threads);
int oracle_fp8_quantize(const float *w, int64_t n, int64_t k, uint8_t *codes, float *row_scales, int threads);
void oracle_fp8_gemm_cols(const uint16_t *a, int64_t m, int64_t k, const uint8_t *codes,
                          const float *row_scales, const int64_t *cols, int64_t ncols, double *c, double *s,
                          int threads);
}

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}
float next_f32() { return ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * 8.0f; }

template <class T>
bool same(const std::vector<T> &x, const std::vector<T> &y) {
  return x.size() == y.size() && std::memcmp(x.data(), y.data(), x.size() * sizeof(T)) == 0;
}

}  // namespace

int main() {
  const int64_t n = 97, k = 256, m = 5;
  std::vector<float> w((size_t)(n * k));
  for (auto &x : w) x = next_f32();
  std::vector<uint16_t> a((size_t)(m * k));
  for (auto &x : a) x = (uint16_t)(0x3C00u | (next_u32() & 0x01FFu) | ((next_u32() & 1u) << 15));

  int bad = 0;
  std::vector<uint8_t> c1((size_t)(n * k / 2)), s1((size_t)(n * k / 16)), c4(c1.size()), s4(s1.size());
  bad |= oracle_quantize(w.data(), n, k, c1.data(), s1.data(), 1) != 0;
  bad |= oracle_quantize(w.data(), n, k, c4.data(), s4.data(), 4) != 0;
  bad |= !same(c1, c4) || !same(s1, s4);

  std::vector<double> g1((size_t)(m * n)), g4(g1.size()), a1(g1.size()), a4(g1.size());
  oracle_gemm(a.data(), m, k, c1.data(), s1.data(), n, 1.0, g1.data(), a1.data(), 1);
  oracle_gemm(a.data(), m, k, c1.data(), s1.data(), n, 1.0, g4.data(), a4.data(), 4);
  bad |= !same(g1, g4) || !same(a1, a4);

  std::vector<uint8_t> f1((size_t)(n * k)), f4(f1.size());
  std::vector<float> r1((size_t)n), r4((size_t)n);
  bad |= oracle_fp8_quantize(w.data(), n, k, f1.data(), r1.data(), 1) != 0;
  bad |= oracle_fp8_quantize(w.data(), n, k, f4.data(), r4.data(), 4) != 0;
  bad |= !same(f1, f4) || !same(r1, r4);

  std::vector<int64_t> cols = {0, 5, 17, 96, 40};
  std::vector<double> h1((size_t)(m * 5)), h4(h1.size());
  oracle_fp8_gemm_cols(a.data(), m, k, f1.data(), r1.data(), cols.data(), 5, h1.data(), nullptr, 1);
  oracle_fp8_gemm_cols(a.data(), m, k, f1.data(), r1.data(), cols.data(), 5, h4.data(), nullptr, 3);
  bad |= !same(h1, h4);

  std::printf(bad ? "MISMATCH\n" : "ok\n");
  return bad ? 1 : 0;
}
