// Host-side argument validation of the C ABI, run under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; nothing here reaches a GPU).
// Every call below is rejected on the host before any HIP call or launch, so
// the pointers it passes (a fake address, never dereferenced) are never used.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gptq.h"

static int failures = 0;

static void expect(bool ok, const char *what) {
  if (!ok) {
    std::printf("FAIL: %s (last error: %s)\n", what, gptq_last_error());
    ++failures;
  }
}

static bool said(const char *word) { return std::strstr(gptq_last_error(), word) != nullptr; }

int main() {
  void *fake = reinterpret_cast<void *>(uintptr_t(0x10000));
  float *ff = static_cast<float *>(fake);
  gptq_params p{4, 128, 128, 1, 0.01f, GPTQ_GRID_AFFINE, 0};

  // workspace sizes
  expect(gptq_workspace_bytes(4096, 11008, &p) >= size_t(11008) * 11008 * 4, "ws d x d");
  expect(gptq_workspace_bytes(0, 11008, &p) == 0, "ws rows 0");
  expect(gptq_workspace_bytes(4096, 11008, nullptr) == 0, "ws params NULL");
  gptq_params bad = p;
  bad.group = 100;
  expect(gptq_workspace_bytes(4096, 11008, &bad) == 0, "ws bad group");

  // parameter checks of gptq_quantize_layer
  const struct { int bits, group, block, act, grid, search; float damp; const char *word; } cases[] = {
      {9, 128, 128, 0, 0, 0, 0.01f, "bits"},   {1, 128, 128, 0, 0, 0, 0.01f, "bits"},
      {4, 128, 0, 0, 0, 0, 0.01f, "block"},    {4, 128, 129, 0, 0, 0, 0.01f, "block"},
      {4, 96, 64, 0, 0, 0, 0.01f, "divide"},   {4, 128, 128, 2, 0, 0, 0.01f, "act_order"},
      {4, 128, 128, 0, 0, 0, -1.f, "percdamp"}, {4, 128, 128, 0, 0, 0, NAN, "percdamp"},
      {7, 256, 128, 0, 1, 0, 0.01f, "[2, 6]"}, {4, 128, 128, 0, 1, 0, 0.01f, "256"},
      {4, 128, 128, 0, 7, 0, 0.01f, "grid"},   {4, 96, 32, 0, 0, 0, 0.01f, "multiple of group"},
      {4, 128, 128, 0, 0, 2, 0.01f, "search"},
  };
  for (const auto &c : cases) {
    gptq_params q{c.bits, c.group, c.block, c.act, c.damp, c.grid, c.search};
    gptq_status st = gptq_quantize_layer(ff, 64, 1024, ff, (int32_t *)fake, (uint8_t *)fake,
                                         (double *)fake, &q, (uint8_t *)fake, (int32_t *)fake, ff,
                                         (uint8_t *)fake, (uint16_t *)fake, (uint16_t *)fake,
                                         (uint8_t *)fake, (uint8_t *)fake, fake, size_t(1) << 30,
                                         nullptr);
    expect(st == GPTQ_ERR_INVALID_ARG && said(c.word), c.word);
  }
  expect(gptq_quantize_layer(nullptr, 64, 1024, ff, (int32_t *)fake, (uint8_t *)fake, nullptr, &p,
                             (uint8_t *)fake, (int32_t *)fake, ff, (uint8_t *)fake, nullptr,
                             nullptr, nullptr, nullptr, fake, size_t(1) << 30,
                             nullptr) == GPTQ_ERR_INVALID_ARG,
         "quantize W NULL");
  expect(gptq_quantize_layer(ff, 64, 1024, ff, (int32_t *)fake, (uint8_t *)fake, nullptr, &p,
                             (uint8_t *)fake, (int32_t *)fake, ff, (uint8_t *)fake, nullptr,
                             nullptr, nullptr, nullptr, fake, 16, nullptr) == GPTQ_ERR_WORKSPACE,
         "quantize ws too small");

  // gptq_hessian_accumulate
  double *dd = static_cast<double *>(fake);
  expect(gptq_hessian_accumulate(nullptr, dd, 16, fake, GPTQ_DT_BF16, 8, 8, nullptr, 0,
                                 nullptr) == GPTQ_ERR_INVALID_ARG, "H NULL");
  expect(gptq_hessian_accumulate(ff, dd, 16, fake, 5, 8, 8, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "x dtype");
  expect(gptq_hessian_accumulate(ff, dd, 16, fake, GPTQ_DT_BF16, 8, 4, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG && said("ld_x"), "ld_x < n");
  expect(gptq_hessian_accumulate(ff, dd, 16, fake, GPTQ_DT_BF16, 12, 12, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "ld_x multiple of 8");
  expect(gptq_hessian_accumulate(ff, dd, 0, fake, GPTQ_DT_BF16, 8, 8, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "d = 0");
  expect(gptq_hessian_accumulate(ff, dd, 16, reinterpret_cast<void *>(uintptr_t(0x10002)),
                                 GPTQ_DT_BF16, 8, 8, nullptr, 0, nullptr) == GPTQ_ERR_INVALID_ARG,
         "X misaligned");
  expect(gptq_hessian_accumulate(ff, dd, 16, fake, GPTQ_DT_BF16, 8, 8,
                                 reinterpret_cast<void *>(uintptr_t(0x10010)), 1 << 20,
                                 nullptr) == GPTQ_ERR_WORKSPACE, "ws misaligned");
  expect(gptq_hessian_accumulate(ff, dd, 16, nullptr, GPTQ_DT_BF16, 0, 0, nullptr, 0, nullptr) ==
             GPTQ_OK, "empty chunk");

  // gptq_prepare_hinv workspace
  int32_t *ip = static_cast<int32_t *>(fake);
  uint8_t *bp = static_cast<uint8_t *>(fake);
  expect(gptq_prepare_hinv(ff, dd, 1024, &p, ff, ip, bp, nullptr, 0, nullptr) ==
             GPTQ_ERR_WORKSPACE, "prepare ws NULL");
  expect(gptq_prepare_hinv(ff, dd, 1024, &p, ff, ip, bp, fake, 10, nullptr) ==
             GPTQ_ERR_WORKSPACE && said("too small"), "prepare ws small");
  expect(gptq_prepare_hinv(ff, dd, 1024, &p, ff, ip, bp,
                           reinterpret_cast<void *>(uintptr_t(0x10010)), size_t(1) << 40,
                           nullptr) == GPTQ_ERR_WORKSPACE && said("aligned"), "prepare ws align");

  // gptq_pack
  uint32_t *up = static_cast<uint32_t *>(fake);
  expect(gptq_pack(bp, 4, 10, 3, up, nullptr) == GPTQ_ERR_INVALID_ARG, "pack 30 bits");
  expect(gptq_pack(bp, 4, 32, 9, up, nullptr) == GPTQ_ERR_INVALID_ARG, "pack bits 9");
  expect(gptq_pack(nullptr, 4, 32, 4, up, nullptr) == GPTQ_ERR_INVALID_ARG, "pack NULL");
  expect(gptq_pack(bp, 0, 32, 4, up, nullptr) == GPTQ_OK, "pack nothing");

  // W4A16
  expect(gptq_w4a16_layer_bytes(4096, 11008, 128) > 0, "w4a16 bytes");
  expect(gptq_w4a16_layer_bytes(4096, 11008, 100) == 0, "w4a16 bytes bad group");
  gptq_w4a16_layer lay{};
  expect(gptq_w4a16_prepare(up, ip, ff, up, 64, 128, 48, fake, size_t(1) << 24, &lay, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "w4a16 prepare group");
  expect(gptq_w4a16_prepare(up, ip, ff, up, 64, 128, 32, fake, 4096, &lay, nullptr) ==
             GPTQ_ERR_INVALID_ARG && said("too small"), "w4a16 prepare mem");
  gptq_w4a16_layer empty{};
  expect(gptq_w4a16_gemm(&empty, (uint16_t *)fake, 1, (uint16_t *)fake, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "w4a16 gemm unprepared");
  gptq_w4a16_layer l2{4096, 11008, 128, 1, 4096, 11008, fake, size_t(1) << 30};
  expect(gptq_w4a16_gemm(&l2, (uint16_t *)fake, 0, (uint16_t *)fake, nullptr, 0, nullptr) ==
             GPTQ_ERR_INVALID_ARG, "w4a16 batch 0");
  expect(gptq_w4a16_gemm(&l2, (uint16_t *)fake, 16, (uint16_t *)fake, nullptr, 0, nullptr) ==
             GPTQ_ERR_WORKSPACE, "w4a16 ws");

  // calibration helpers
  expect(gptq_linear_forward_ws_bytes(0, 16, 16) == 0, "forward ws bytes");
  expect(gptq_linear_forward(nullptr, 16, 16, (uint16_t *)fake, 16, 16, (uint16_t *)fake, 16,
                             fake, size_t(1) << 20, nullptr) == GPTQ_ERR_INVALID_ARG,
         "forward W NULL");

  // profiler
  int64_t n = -1;
  double ms = -1;
  expect(gptq_profile_query("no_such_kernel", &n, &ms) == GPTQ_OK && n == 0 && ms == 0.0,
         "profile unknown");
  expect(gptq_profile_query(nullptr, &n, &ms) == GPTQ_ERR_INVALID_ARG, "profile NULL");

  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
