// Host-side exercise of libqlinear's C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: packing, unpacking and the RTN fit on the CPU,
// argument validation of the device entry points (every call here returns
// before any device work), sizing queries, status strings and the last-path
// buffer. Buffers are allocated at their exact sizes so any overrun is
// reported. Exit status 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "qlinear.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

static void pack_round_trips(std::mt19937 &rng) {
  for (int bits : {2, 3, 4, 8}) {
    for (int64_t N : {1, 3, 7}) {
      for (int64_t K : {64, 128, 320}) {
        std::vector<uint8_t> q(N * K), back(N * K);
        for (auto &v : q) v = (uint8_t)(rng() % (1u << bits));
        std::vector<uint32_t> words(qlinear_packed_words(bits, N, K));
        CHECK(words.size() == (size_t)(N * K * bits / 32));
        CHECK(qlinear_pack_host(q.data(), bits, N, K, words.data()) == QL_OK);
        CHECK(qlinear_unpack_host(words.data(), bits, N, K, back.data()) == QL_OK);
        CHECK(q == back);
      }
    }
    // a code out of range is refused
    std::vector<uint8_t> q(64, 0);
    q[17] = (uint8_t)(1u << bits);
    std::vector<uint32_t> words(qlinear_packed_words(bits, 1, 64));
    if (bits < 8) CHECK(qlinear_pack_host(q.data(), bits, 1, 64, words.data()) == QL_ERANGE);
  }
  CHECK(qlinear_pack_host(nullptr, 4, 1, 64, nullptr) != QL_OK);
  CHECK(qlinear_pack_host(nullptr, 5, 1, 64, nullptr) != QL_OK);
}

static float f16_value(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  const float v = e == 0 ? std::ldexp((float)m, -24) : e == 31 ? INFINITY : std::ldexp((float)(m | 1024), e - 25);
  return (h & 0x8000) ? -v : v;
}

static void rtn_fits(std::mt19937 &rng) {
  std::normal_distribution<float> nd(0.f, 0.02f);
  for (int bits : {2, 3, 4, 8}) {
    const int64_t N = 5, K = 192, G = K / 64;
    std::vector<float> w(N * K);
    for (auto &v : w) v = nd(rng);
    for (int64_t k = 0; k < 64; ++k) w[64 + k] = 0.25f;   // a constant group
    w[2 * K + 3] = -0.f;
    std::vector<uint8_t> q(N * K);
    std::vector<uint16_t> s(N * G), b(N * G);
    CHECK(qlinear_quantize_rtn_host(w.data(), bits, 64, N, K, q.data(), s.data(), b.data()) == QL_OK);
    for (auto v : q) CHECK(v < (1u << bits));
    // each weight within half a step of its dequantized value (plus f16 rounding of s and b)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const float sc = f16_value(s[n * G + k / 64]), bi = f16_value(b[n * G + k / 64]);
        const float wh = sc * (float)q[n * K + k] + bi;
        CHECK(std::fabs(wh - w[n * K + k]) <= 0.5f * sc + 1e-3f * std::fabs(w[n * K + k]) + 1e-6f);
      }
    // non-finite and overflowing inputs are refused
    std::vector<float> bad = w;
    bad[5] = NAN;
    CHECK(qlinear_quantize_rtn_host(bad.data(), bits, 64, N, K, q.data(), s.data(), b.data()) == QL_ERANGE);
    bad[5] = -1e5f;  // the group minimum, its f16 bias, overflows
    CHECK(qlinear_quantize_rtn_host(bad.data(), bits, 64, N, K, q.data(), s.data(), b.data()) == QL_ERANGE);
    CHECK(qlinear_quantize_rtn_host(w.data(), bits, 32, N, K, q.data(), s.data(), b.data()) != QL_OK);
  }
}

static void validation_and_sizes() {
  // sizes
  for (int bits : {2, 3, 4, 8})
    for (int64_t M : {1, 16, 17, 300, 4096})
      for (int64_t N : {32, 264, 4608})
        for (int64_t K : {64, 4608}) {
          const size_t ws = qlinear_workspace_bytes(bits, M, N, K);
          ql_forward_args a;
          std::memset(&a, 0, sizeof(a));
          a.x = (const void *)0x1000;
          a.packed_q = (const uint32_t *)0x2000;
          a.scales = (const void *)0x3000;
          a.biases = (const void *)0x4000;
          a.out = (void *)0x5000;
          a.bits = bits;
          a.group = 64;
          a.M = M;
          a.N = N;
          a.K = K;
          for (int mode : {QL_MODE_AUTO, QL_MODE_EXACT, QL_MODE_FAST, QL_MODE_SPLIT}) {
            a.mode = mode;
            CHECK(qlinear_forward_workspace_bytes(&a) <= ws);
          }
          CHECK(qlinear_tiled_words(bits, N, K) >= qlinear_packed_words(bits, N, K));
        }
  CHECK(qlinear_workspace_bytes(5, 10, 10, 64) == 0);
  CHECK(qlinear_workspace_bytes(4, 10, 10, 65) == 0);
  CHECK(qlinear_tiled_sb_words(33, 128) == 64 * 2);
  CHECK(qlinear_forward_noalloc_max_scratch() > 0);
  // forward: every invalid request is refused before any device work
  ql_forward_args a;
  std::memset(&a, 0, sizeof(a));
  a.bits = 4;
  a.group = 64;
  a.M = 4;
  a.N = 8;
  a.K = 64;
  CHECK(qlinear_forward_ex(&a, nullptr) == QL_EINVAL);  // null pointers
  CHECK(qlinear_forward_ex(nullptr, nullptr) == QL_EINVAL);
  a.x = (const void *)0x1000;
  a.packed_q = (const uint32_t *)0x2000;
  a.scales = (const void *)0x3000;
  a.biases = (const void *)0x4000;
  a.out = (void *)0x5000;
  a.K = 100;
  CHECK(qlinear_forward_ex(&a, nullptr) == QL_EINVAL);
  a.K = 64;
  a.bits = 5;
  CHECK(qlinear_forward_ex(&a, nullptr) != QL_OK);
  a.bits = 4;
  a.out_dtype = 9;
  CHECK(qlinear_forward_ex(&a, nullptr) == QL_EINVAL);
  a.out_dtype = 0;
  a.x = (const void *)0x1004;
  CHECK(qlinear_forward_ex(&a, nullptr) == QL_EALIGN);
  a.x = (const void *)0x1000;
  a.M = 0;
  CHECK(qlinear_forward_ex(&a, nullptr) == QL_OK);  // empty: no-op
  CHECK(qlinear_forward(nullptr, nullptr, nullptr, nullptr, 4, 64, 0, 8, 64, nullptr) == QL_OK);
  CHECK(qlinear_forward(nullptr, nullptr, nullptr, nullptr, 4, 32, 4, 8, 64, nullptr) != QL_OK);
  // device entry points' argument checks
  CHECK(qlinear_dequantize((const uint32_t *)0x1000, (const void *)0x2000, (const void *)0x3000, 4, 64, 4, 65,
                           (float *)0x4000, nullptr) == QL_EINVAL);
  CHECK(qlinear_fast_activations(nullptr, 4, 64, nullptr, nullptr, nullptr) == QL_EINVAL);
  CHECK(qlinear_fast_activations_adaln((const void *)0x1000, (const float *)0x2004, 1, 4, 64, (void *)0x3000,
                                       (float *)0x4000, nullptr) == QL_EALIGN);
  CHECK(qlinear_group_sums((const void *)0x1000, 4, 64, (float *)0x2000, 1, nullptr) == QL_EINVAL);
  CHECK(qlinear_repack(nullptr, nullptr, nullptr, 4, 64, 8, 64, nullptr, nullptr, nullptr) == QL_EINVAL);
}

static void strings() {
  for (int st = -12; st <= 4; ++st) {
    const char *s = qlinear_status_string(st);
    CHECK(s != nullptr && std::strlen(s) > 0);
  }
  std::vector<char> tiny(1), big(256);
  CHECK(qlinear_last_path(tiny.data(), tiny.size()) == QL_OK && tiny[0] == '\0');
  CHECK(qlinear_last_path(big.data(), big.size()) == QL_OK && std::strlen(big.data()) < big.size());
  CHECK(qlinear_last_path(nullptr, 8) == QL_EINVAL);
  CHECK(qlinear_last_path(big.data(), 0) == QL_EINVAL);
  CHECK(qlinear_version() >= 100);
}

int main() {
  std::mt19937 rng(1234);
  pack_round_trips(rng);
  rtn_fits(rng);
  validation_and_sizes();
  strings();
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
