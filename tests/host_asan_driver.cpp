// Host-side driver of the C ABI for the sanitizer build (test_host_asan.py).
// It runs the library's host code only: configuration and size queries,
// handle creation and destruction, weight binding with r = 0 (no launch),
// and every compute entry point with one argument out of range, so that each
// returns its error before anything is enqueued.  Pointers are aligned
// stand-ins that the validation never dereferences.  Exit status 0 and a
// final "ALL OK" when every call returned what it should; the sanitizers
// abort the process on a memory error, and leak detection runs at exit.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "ttq.h"

namespace {

std::atomic<int> failures{0};

void expect(const char* what, ttq_status got, ttq_status want) {
  const char* msg = ttq_last_error();
  const size_t len = std::strlen(msg);  // the message must be a terminated string
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, msg);
    ++failures;
  } else if (want != TTQ_OK && len == 0) {
    std::printf("FAIL %s: error without a message\n", what);
    ++failures;
  }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t(1) << 20) + off); }

ttq_config cfg(int d_in, int d_out, int q, int g, int r) { return ttq_config{d_in, d_out, q, g, r, 0.5f, 0.4f, 2.0f}; }

ttq_buffers buffers(int64_t T_max, bool lowrank, size_t ws) {
  ttq_buffers b{};
  b.codes = static_cast<uint32_t*>(fake());
  b.scales = fake();
  b.zeros = fake();
  b.D = static_cast<float*>(fake());
  b.dinvsqrt = static_cast<float*>(fake());
  b.wres = lowrank ? fake() : nullptr;
  b.B = lowrank ? static_cast<const float*>(fake()) : nullptr;
  b.A = lowrank ? static_cast<const float*>(fake()) : nullptr;
  b.workspace = static_cast<float*>(fake());
  b.T_max = T_max;
  b.workspace_bytes = ws;
  b.wexp = nullptr;
  return b;
}

void config_and_sizes() {
  ttq_sizes sz;
  ttq_config c = cfg(5120, 8192, 4, 32, 0);
  expect("query_sizes", ttq_query_sizes(&c, 16384, &sz), TTQ_OK);
  expect("query_sizes NULL cfg", ttq_query_sizes(nullptr, 16, &sz), TTQ_ERR_NULL);
  expect("query_sizes NULL out", ttq_query_sizes(&c, 16, nullptr), TTQ_ERR_NULL);
  const int qs[] = {1, 6, 8, -3};
  for (int q : qs) {
    ttq_config b = cfg(5120, 8192, q, 32, 0);
    expect("query_sizes q", ttq_query_sizes(&b, 16, &sz), TTQ_ERR_INVALID_ARG);
  }
  ttq_config g8 = cfg(5120, 8192, 4, 8, 0);
  expect("query_sizes g=8", ttq_query_sizes(&g8, 16, &sz), TTQ_ERR_UNSUPPORTED);
  ttq_config din = cfg(100, 8192, 4, 32, 0);
  expect("query_sizes d_in", ttq_query_sizes(&din, 16, &sz), TTQ_ERR_SHAPE);
  ttq_config big = cfg(1 << 22, 8192, 4, 32, 0);
  expect("query_sizes d_in 2^22", ttq_query_sizes(&big, 16, &sz), TTQ_ERR_SHAPE);
  ttq_config nan = cfg(5120, 8192, 4, 32, 0);
  nan.alpha = __builtin_nanf("");
  expect("query_sizes alpha NaN", ttq_query_sizes(&nan, 16, &sz), TTQ_ERR_INVALID_ARG);
  for (int s = -1; s < 9; ++s) {
    const char* t = ttq_status_string(static_cast<ttq_status>(s));
    if (t == nullptr || std::strlen(t) == 0) {
      std::printf("FAIL status string %d\n", s);
      ++failures;
    }
  }
  const int64_t Ts[] = {0, 1, 4, 5, 64, 65, 16384, int64_t(1) << 40};
  for (int64_t T : Ts) {
    (void)ttq_linear_workspace_bytes(T, 5120, 8192, 0);
    (void)ttq_linear_workspace_bytes(T, 5120, 8192, 16);
    (void)ttq_prefill_workspace_bytes(T, 5120, 8192, 16, TTQ_F16);
    (void)ttq_colstats_workspace_bytes(T, 5120);
  }
  (void)ttq_lowrank_refresh_workspace_bytes(8192, 5120, 16);
  (void)ttq_dense_min_tokens(8192);
  (void)ttq_dense_min_tokens(-5);
}

void handles() {
  // many create / destroy pairs: nothing may leak
  for (int i = 0; i < 64; ++i) {
    ttq_config c = cfg(128, 64, 2 + i % 4, 32, (i & 1) ? 16 : 0);
    ttq_buffers b = buffers(16, (i & 1) != 0, size_t(1) << 30);
    ttq_handle* h = nullptr;
    expect("create", ttq_create(&c, &b, &h), TTQ_OK);
    if (!(i & 1)) {
      expect("set_weight r=0", ttq_set_weight(h, fake(), nullptr), TTQ_OK);
      expect("prepare T>T_max", ttq_prepare(h, fake(), TTQ_F16, 17, 128, nullptr), TTQ_ERR_SHAPE);
      expect("prepare NULL X", ttq_prepare(h, nullptr, TTQ_F16, 4, 128, nullptr), TTQ_ERR_NULL);
      expect("prepare ldx", ttq_prepare(h, fake(), TTQ_F16, 4, 130, nullptr), TTQ_ERR_ALIGN);
      expect("linear before prepare", ttq_linear(h, fake(), TTQ_F16, 4, 128, fake(), 64, fake(), 1 << 20, nullptr),
             TTQ_ERR_INVALID_ARG);
      expect("prefill T=0", ttq_prefill(h, fake(), TTQ_F16, 0, 128, fake(), 64, fake(), 1 << 20, nullptr),
             TTQ_ERR_SHAPE);
    } else {
      expect("prepare unbound", ttq_prepare(h, fake(), TTQ_F16, 4, 128, nullptr), TTQ_ERR_INVALID_ARG);
      expect("prepare_refresh unbound",
             ttq_prepare_refresh(h, fake(), TTQ_F16, 4, 128, nullptr, fake(), 1 << 30, nullptr), TTQ_ERR_INVALID_ARG);
    }
    ttq_destroy(h);
  }
  ttq_destroy(nullptr);
  ttq_handle* h = nullptr;
  ttq_config c = cfg(128, 64, 4, 32, 0);
  ttq_buffers small = buffers(16, false, 4);
  expect("create small workspace", ttq_create(&c, &small, &h), TTQ_ERR_SHAPE);
  ttq_buffers nob = buffers(16, false, size_t(1) << 30);
  nob.codes = nullptr;
  expect("create NULL codes", ttq_create(&c, &nob, &h), TTQ_ERR_NULL);
  ttq_buffers mis = buffers(16, false, size_t(1) << 30);
  mis.scales = fake(4);
  expect("create misaligned scales", ttq_create(&c, &mis, &h), TTQ_ERR_ALIGN);
  ttq_config c16 = cfg(128, 64, 4, 32, 16);
  ttq_buffers nolr = buffers(16, false, size_t(1) << 30);
  expect("create r=16 without factors", ttq_create(&c16, &nolr, &h), TTQ_ERR_NULL);
  expect("set_weight NULL handle", ttq_set_weight(nullptr, fake(), nullptr), TTQ_ERR_NULL);
  expect("linear NULL handle", ttq_linear(nullptr, fake(), TTQ_F16, 4, 128, fake(), 64, fake(), 1, nullptr),
         TTQ_ERR_NULL);
}

void sub_steps() {
  void* P = fake();
  float* F = static_cast<float*>(fake());
  uint32_t* U = static_cast<uint32_t*>(fake());
  expect("colstats ldx", ttq_colstats(P, TTQ_F16, 4, 128, 130, 2.f, .4f, .5f, F, F, F, 1 << 20, nullptr),
         TTQ_ERR_ALIGN);
  expect("colstats T=0", ttq_colstats(P, TTQ_F16, 0, 128, 128, 2.f, .4f, .5f, F, F, F, 1 << 20, nullptr),
         TTQ_ERR_SHAPE);
  expect("colstats dtype", ttq_colstats(P, static_cast<ttq_dtype>(9), 4, 128, 128, 2.f, .4f, .5f, F, F, F, 1 << 20,
                                        nullptr),
         TTQ_ERR_INVALID_ARG);
  expect("colstats_noalloc d", ttq_colstats_noalloc(P, TTQ_F16, 64, 16448, 16448, 2.f, .4f, .5f, F, F, nullptr),
         TTQ_ERR_SHAPE);
  expect("quantize_pack NULL W", ttq_quantize_pack(64, 128, 4, 32, nullptr, F, U, P, P, nullptr), TTQ_ERR_NULL);
  expect("quantize_pack d_out", ttq_quantize_pack(40, 128, 4, 32, P, F, U, P, P, nullptr), TTQ_ERR_SHAPE);
  expect("residual r", ttq_residual(64, 128, 8, P, F, F, P, nullptr), TTQ_ERR_UNSUPPORTED);
  expect("lowrank_z r", ttq_lowrank_z(4, 128, 0, P, TTQ_F16, 128, F, F, nullptr), TTQ_ERR_INVALID_ARG);
  expect("prescale d", ttq_prescale(P, TTQ_F16, 4, 96, 96, F, P, nullptr), TTQ_ERR_SHAPE);
  expect("wlowbit_gemm ldy", ttq_wlowbit_gemm(8, 128, 64, 4, 32, 0, P, 128, U, P, P, nullptr, nullptr, P, TTQ_F16,
                                              32, nullptr),
         TTQ_ERR_SHAPE);
  expect("wlowbit_gemm_raw T", ttq_wlowbit_gemm_raw(64, 128, 64, 4, 32, 0, P, 128, P, U, P, P, nullptr, nullptr, P, 64,
                                                    nullptr),
         TTQ_ERR_SHAPE);
  expect("wexp_gemm NULL W", ttq_wexp_gemm(300, 128, 64, 0, P, 128, nullptr, nullptr, nullptr, P, 64, nullptr),
         TTQ_ERR_NULL);
  expect("lowrank_refresh d_in", ttq_lowrank_refresh(64, 192, 16, P, F, F, F, F, P, 1 << 30, nullptr),
         TTQ_ERR_SHAPE);
  expect("lowrank_refresh ws", ttq_lowrank_refresh(64, 256, 16, P, F, F, F, F, P, 16, nullptr), TTQ_ERR_SHAPE);
  // a long message: the formatting must stay inside its buffer
  expect("colstats huge ldx", ttq_colstats(P, TTQ_F16, 4, 128, int64_t(1) << 62, 2.f, .4f, .5f, F, F, F, 1 << 20,
                                           nullptr),
         TTQ_ERR_SHAPE);
}

}  // namespace

int main() {
  config_and_sizes();
  handles();
  sub_steps();
  // the error message is per thread
  std::vector<std::thread> th;
  for (int i = 0; i < 4; ++i)
    th.emplace_back([] {
      for (int k = 0; k < 200; ++k) sub_steps();
    });
  for (auto& t : th) t.join();
  if (failures) {
    std::printf("%d FAILED\n", failures.load());
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
