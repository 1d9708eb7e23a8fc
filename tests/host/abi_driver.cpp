// Host-side checks of libkdloss's argument validation and workspace planning,
// built with the address and undefined-behaviour sanitizers on the host code
// (the kernels are not instrumented, and no call here reaches the GPU: every
// call is rejected, or sizes a workspace, before its first HIP call).
// Prints one line per failed expectation and exits nonzero if there is any.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "kdloss.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::printf("FAILED line %d: %s (last error: %s)\n", line, what, kd_last_error());
    ++failures;
  }
}
#define EXPECT(x) expect((x), #x, __LINE__)

// an aligned address that is never dereferenced: every call below fails or
// returns before touching memory
void* const F = reinterpret_cast<void*>(uintptr_t(0x10000));
template <class T>
T* f(uintptr_t off = 0) {
  return reinterpret_cast<T*>(uintptr_t(0x10000) + off);
}

kd_status topk_fwd(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt, float tau, size_t wsb, const void* H = F,
                   float* kl = f<float>(), void* ws = F) {
  return kd_topk_kl_fwd(H, F, f<int32_t>(), f<float>(), nullptr, tau, T, d, V, K, dt, kl, f<float>(), nullptr, ws,
                        wsb, nullptr);
}

size_t ws_topk(int64_t T, int64_t d, int64_t V, int64_t K, kd_dtype dt, int64_t chunk) {
  size_t b = 0;
  EXPECT(kd_topk_kl_workspace_size(T, d, V, K, dt, chunk, &b) == KD_OK);
  return b;
}

}  // namespace

int main() {
  // rejections of the forward, before any launch
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, 1.f, 0) == KD_ERR_WORKSPACE_TOO_SMALL);
  EXPECT(topk_fwd(-1, 64, 256, 4, KD_BF16, 1.f, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 0, KD_BF16, 1.f, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 257, KD_BF16, 1.f, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 1 << 20, KD_MAX_K + 1, KD_BF16, 1.f, 0) == KD_ERR_UNSUPPORTED);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, 0.f, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, std::nanf(""), 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, INFINITY, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 60, 256, 4, KD_BF16, 1.f, 0) == KD_ERR_UNSUPPORTED);
  EXPECT(topk_fwd(8, 64, 260, 4, KD_BF16, 1.f, 0) == KD_ERR_UNSUPPORTED);
  EXPECT(topk_fwd(8, 64, 256, 4, (kd_dtype)7, 1.f, 0) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, 1.f, 0, f<char>(8)) == KD_ERR_ALIGNMENT);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, 1.f, 0, F, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(topk_fwd(8, 64, 256, 4, KD_BF16, 1.f, 1 << 30, F, f<float>(), f<char>(128)) == KD_ERR_ALIGNMENT);
  EXPECT(topk_fwd(int64_t(1) << 31, 64, 256, 4, KD_BF16, 1.f, 0) == KD_ERR_UNSUPPORTED);
  EXPECT(topk_fwd(0, 64, 256, 4, KD_BF16, 1.f, 0, nullptr, nullptr, nullptr) == KD_OK);  // T = 0: a no-op

  // the backward and the single call
  EXPECT(kd_topk_kl_bwd(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, 8, 64, 256, 4, KD_BF16, f<float>(), f<float>(),
                        F, nullptr, 0, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_topk_kl_bwd(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, 8, 64, 256, 4, KD_BF16, f<float>(), f<float>(),
                        F, f<float>(), -1, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_topk_kl_fwd_bwd(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, 8, 64, 256, 4, KD_BF16, f<float>(),
                            f<float>(), f<float>(), nullptr, F, f<float>(4), 0, F, 0, nullptr) == KD_ERR_ALIGNMENT);

  // options
  kd_topk_opts o{};
  o.ce_weight = 0.5f;  // without labels
  EXPECT(kd_topk_kl_fwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                           f<float>(), nullptr, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  o = kd_topk_opts{};
  o.rev_weight = -0.5f;  // outside [0, 1]
  EXPECT(kd_topk_kl_fwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                           f<float>(), f<float>(), F, 0, nullptr) == KD_ERR_INVALID_ARG);
  o.rev_weight = 0.5f;  // without z_topk: the forward, the backward and the single call
  EXPECT(kd_topk_kl_fwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                           f<float>(), nullptr, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_topk_kl_bwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                           f<float>(), F, f<float>(), 0, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_topk_kl_fwd_bwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                               f<float>(), f<float>(), nullptr, F, f<float>(), 0, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  o.z_topk = f<float>(2);  // misaligned
  EXPECT(kd_topk_kl_bwd_ex(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 4, KD_BF16, f<float>(),
                           f<float>(), F, f<float>(), 0, F, 0, nullptr) == KD_ERR_ALIGNMENT);
  o.z_topk = f<float>();  // a shard cannot form the reverse part
  EXPECT(kd_topk_kl_fwd_shard(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 512, 4, KD_BF16,
                              f<float>(), f<float>(), f<float>(), F, 0, nullptr) == KD_ERR_UNSUPPORTED);
  o = kd_topk_opts{};
  o.check_indices = 1;
  EXPECT(kd_topk_kl_fwd_shard(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, &o, 8, 64, 256, 512, 4, KD_BF16,
                              f<float>(), f<float>(), nullptr, F, 0, nullptr) == KD_ERR_UNSUPPORTED);
  kd_full_opts fo{};
  fo.rev_weight = 2.f;
  EXPECT(kd_full_kl_fwd_ex(F, F, F, F, nullptr, 1.f, &fo, 8, 64, 64, 256, KD_BF16, f<float>(), f<float>(), f<float>(),
                           nullptr, F, 0, nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_full_kl_shard_combine(f<float>(), 0, nullptr, 8, 0.f, f<float>(), f<float>(), f<float>(), nullptr,
                                  nullptr) == KD_ERR_INVALID_ARG);
  EXPECT(kd_topk_kl_shard_combine(f<float>(), 4, f<float>(), nullptr, int64_t(1) << 30, f<float>(), f<float>(),
                                  nullptr) == KD_ERR_UNSUPPORTED);

  // the forward without a workspace refuses shapes beyond its scratch on the host
  EXPECT(kd_topk_kl_fwd_noalloc(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, 200000, 3072, 128256, 64, KD_BF16,
                                f<float>(), f<float>(), nullptr, nullptr) == KD_ERR_UNSUPPORTED);

  // workspace planning across shapes: affine in T for a fixed chunk, never a
  // [T, V] buffer, every size query consistent with the call's own check
  const int64_t Ts[] = {1, 255, 256, 257, 4096, 4097, 65536, 262144, int64_t(1) << 24};
  const int64_t Ks[] = {1, 64, 100, 8192};
  for (int64_t T : Ts)
    for (int64_t K : Ks) {
      if (T * (K + 1) >= std::numeric_limits<int32_t>::max()) continue;
      for (int64_t chunk : {int64_t(0), int64_t(256), int64_t(16384), int64_t(1) << 40}) {
        const size_t b = ws_topk(T, 3072, 128256, K, KD_BF16, chunk);
        EXPECT(b > 0);
        EXPECT(b < size_t(T) * 128256 * 2 + (size_t(5) << 30));
        size_t b2 = 0;
        EXPECT(kd_topk_kl_fwd_bwd_workspace_size(T, 3072, 128256, K, KD_BF16, chunk, &b2) == KD_OK && b2 >= b);
        EXPECT(kd_full_kl_workspace_size(T, 3072, 4096, 128256, KD_BF16, chunk, &b2) == KD_OK && b2 > 0);
        EXPECT(kd_full_kl_fwd_bwd_workspace_size(T, 3072, 4096, 128256, KD_BF16, chunk, &b2) == KD_OK && b2 > 0);
        EXPECT(kd_topk_kl_shard_workspace_size(T, 3072, 16032, 16032, K, KD_BF16, chunk, &b2) == KD_OK && b2 > 0);
      }
    }
  {
    const size_t a = ws_topk(65536, 3072, 128256, 64, KD_BF16, 0), b = ws_topk(262144, 3072, 128256, 64, KD_BF16, 0);
    const double slope = double(b - a) / (262144 - 65536);
    EXPECT(slope > 0 && slope <= 1024);
  }
  // the size query serves both calls; the backward needs all of it, so one
  // byte short is refused before any launch
  {
    const size_t b = ws_topk(8, 64, 256, 4, KD_BF16, 0);
    EXPECT(kd_topk_kl_bwd(F, F, f<int32_t>(), f<float>(), nullptr, 1.f, 8, 64, 256, 4, KD_BF16, f<float>(),
                          f<float>(), F, f<float>(), 0, F, b - 1, nullptr) == KD_ERR_WORKSPACE_TOO_SMALL);
  }
  for (int s = 0; s <= 7; ++s) EXPECT(kd_status_string((kd_status)s) != nullptr);
  EXPECT(kd_version() > 0);

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
