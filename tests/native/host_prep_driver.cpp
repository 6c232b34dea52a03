// Drives the host-side entry points of libsvdq (prep, LoRA concat, smoothing,
// argument errors) on small seeded inputs. Built with g++ and
// -fsanitize=address,undefined by tests/test_host_sanitize.py; no GPU code.
#include <cmath>
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>

#include "../../include/svdq.h"

static int fail(const char* what) {
  std::fprintf(stderr, "FAIL: %s (%s)\n", what, svdq_last_error());
  return 1;
}

int main() {
  std::mt19937_64 rng(42);
  std::normal_distribution<float> nd(0.f, 1.f);
  const int64_t shapes[][3] = {{64, 16, 0}, {128, 96, 16}, {192, 320, 32}, {256, 64, 48}};
  for (auto& s : shapes) {
    const int64_t K = s[0], N = s[1];
    const int32_t r = static_cast<int32_t>(s[2]);
    std::vector<float> X(32 * K), W(K * N), xa(K), lam(K), inv(K);
    for (auto& v : X) v = nd(rng);
    for (auto& v : W) v = 0.02f * nd(rng);
    if (svdq_channel_absmax(X.data(), SVDQ_F32, 32, K, K, xa.data()) != SVDQ_OK) return fail("absmax");
    if (svdq_smoothing_factors(xa.data(), W.data(), K, N, lam.data()) != SVDQ_OK) return fail("lambda");
    std::vector<uint16_t> L1t(r * K + 1), L2t(N * r + 1), ws(N * (K / 64));
    std::vector<uint8_t> wc(N * K / 2);
    std::vector<double> sig(K < N ? K : N);
    if (svdq_prepare_weights(W.data(), lam.data(), K, N, r, 64, inv.data(), L1t.data(), L2t.data(),
                             wc.data(), ws.data(), sig.data()) != SVDQ_OK)
      return fail("prepare");
    for (size_t i = 1; i < sig.size(); ++i)
      if (!(sig[i] <= sig[i - 1] * (1 + 1e-12) + 1e-300)) return fail("sigma order");
    const int32_t rl = 8;
    std::vector<uint16_t> A(K * rl, 0x2000), B(rl * N, 0xA000), L1o((r + rl) * K), L2o(N * (r + rl));
    if (svdq_concat_lora(r ? L1t.data() : nullptr, r ? L2t.data() : nullptr, K, N, r, lam.data(),
                         A.data(), B.data(), rl, 0.5f, L1o.data(), L2o.data()) != SVDQ_OK)
      return fail("lora");
  }
  // argument errors must not touch memory
  if (svdq_prepare_weights(nullptr, nullptr, 64, 8, 0, 64, nullptr, nullptr, nullptr, nullptr,
                           nullptr, nullptr) != SVDQ_ERR_NULL)
    return fail("null check");
  std::puts("host prep driver: ok");
  return 0;
}
