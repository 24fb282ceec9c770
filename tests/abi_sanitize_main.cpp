// Host-only driver of the C ABI's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/sanitize_abi.py): every call below is rejected before any
// HIP call, so no GPU is needed.  Prints one line per failed expectation and "abi-sanitize ok"
// at the end.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kvc.h"

static int g_fail = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, kvc_last_error());
    ++g_fail;
  }
}

int main() {
  char* P = reinterpret_cast<char*>(0x10000);  // 16-byte aligned, never dereferenced
  const float* F = reinterpret_cast<const float*>(P);
  // kvc_correct: shapes, pointers, anchors, workspace
  expect(kvc_correct(nullptr, P, 2, 2, 64, 128, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     1 << 30, nullptr),
         KVC_ERR_ARG, "correct: K NULL");
  expect(kvc_correct(P, P, 2, 2, 64, 96, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     1 << 30, nullptr),
         KVC_ERR_UNSUPPORTED, "correct: d = 96");
  expect(kvc_correct(P, P, 2, 2, 64, 128, KVC_BF16, F, P, P, 9, 32, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     1 << 30, nullptr),
         KVC_ERR_UNSUPPORTED, "correct: A * r > 256");
  expect(kvc_correct(P, P, 2, 2, 64, 128, KVC_F32, F, P, P, 1, 129, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     1 << 30, nullptr),
         KVC_ERR_ARG, "correct: r > d");
  expect(kvc_correct(P, P, 2, 2, 64, 128, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr, P, nullptr,
                     P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P, 1 << 30,
                     nullptr),
         KVC_ERR_ARG, "correct: K_fb without V_fb");
  expect(kvc_correct(P, P, 2, 2, 64, 128, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     16, nullptr),
         KVC_ERR_WORKSPACE, "correct: workspace too small");
  expect(kvc_correct(P, P, 40000, 40000, 64, 128, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr,
                     nullptr, nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr,
                     nullptr, P, 1 << 30, nullptr),
         KVC_ERR_UNSUPPORTED, "correct: L * H overflow");
  expect(kvc_correct(P, P, -1, 2, 64, 128, KVC_BF16, F, P, P, 4, 32, 0.3f, nullptr, nullptr,
                     nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr, nullptr, P,
                     1 << 30, nullptr),
         KVC_ERR_ARG, "correct: negative L");
  // chain / fanout: host arrays
  const float* descs[2] = {F, F};
  const void* facs[2] = {P, P};
  void* outs[2] = {P + 4096, P + 8192};
  uint8_t* masks[2] = {reinterpret_cast<uint8_t*>(P), reinterpret_cast<uint8_t*>(P)};
  expect(kvc_correct_chain(P, P, 2, 2, 64, 128, KVC_BF16, 0, descs, facs, facs, 4, 32, 0.3f,
                           nullptr, nullptr, outs, outs, masks, nullptr, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "chain: no edges");
  expect(kvc_correct_chain(P, P, 2, 2, 64, 128, KVC_BF16, 2, nullptr, facs, facs, 4, 32, 0.3f,
                           nullptr, nullptr, outs, outs, masks, nullptr, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "chain: desc array NULL");
  void* same[2] = {P, P};
  expect(kvc_correct_chain(P, P, 2, 2, 64, 128, KVC_BF16, 1, descs, facs, facs, 4, 32, 0.3f,
                           nullptr, nullptr, same, same, masks, nullptr, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "chain: edge writes over its source");
  expect(kvc_correct_fanout(P, P, 2, 2, 64, 128, KVC_BF16, 2, descs, facs, facs, 4, 32, 0.3f,
                            nullptr, nullptr, same, outs, masks, nullptr, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "fanout: output overlaps the reference");
  // fit and the streaming fit
  int32_t* K32 = reinterpret_cast<int32_t*>(P);
  float* Fo = reinterpret_cast<float*>(P);
  expect(kvc_fit_anchor(P, 4, 64, 128, KVC_BF16, 0, 0.9, Fo, Fo, K32, nullptr, P, 1 << 30,
                        nullptr),
         KVC_ERR_ARG, "fit: r = 0");
  expect(kvc_fit_anchor(P, 4, 64, 128, KVC_BF16, 32, 1.5, Fo, Fo, K32, nullptr, P, 1 << 30,
                        nullptr),
         KVC_ERR_ARG, "fit: energy > 1");
  expect(kvc_fit_anchor(P, 4, 64, 128, KVC_BF16, 32, 0.9, Fo, Fo, K32, nullptr, nullptr, 0,
                        nullptr),
         KVC_ERR_WORKSPACE, "fit: no workspace");
  expect(kvc_fit_from_gram(reinterpret_cast<const double*>(P), 4, 128, 200, 0.9, Fo, K32,
                           nullptr, nullptr),
         KVC_ERR_ARG, "fit_from_gram: r > d");
  expect(kvc_refit_warm(reinterpret_cast<const double*>(P), 4, 128, 0, 0.9, F, Fo, K32, nullptr,
                        nullptr),
         KVC_ERR_ARG, "refit_warm: r = 0");
  expect(kvc_refit_warm(reinterpret_cast<const double*>(P), 4, 128, 32, 0.9, nullptr, Fo, K32,
                        nullptr, nullptr),
         KVC_ERR_ARG, "refit_warm: no W_prev");
  expect(kvc_gram_accumulate(P, 4, -3, 128, KVC_BF16, reinterpret_cast<double*>(P), P, 1 << 30,
                             nullptr),
         KVC_ERR_ARG, "gram: negative T");
  expect(kvc_project(P, 4, 64, 128, KVC_BF16, F, 0, Fo, P, 1 << 30, nullptr), KVC_ERR_ARG,
         "project: r = 0");
  // anchor pool, errors, ranks
  expect(kvc_correct_pooled(P, P, 2, 2, 64, 128, KVC_BF16, F, P, P, K32, 4, 5, 32, 0.3f, nullptr,
                            nullptr, nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr,
                            nullptr, nullptr, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "pooled: A > capacity");
  expect(kvc_anchor_pool_insert(reinterpret_cast<uint8_t*>(P), F, F, F, 2, 2, 64, 128, KVC_BF16,
                                40, 32, P, P, Fo, K32, K32, nullptr),
         KVC_ERR_UNSUPPORTED, "insert: capacity 40");
  expect(kvc_segment_error(P, nullptr, 2, 2, 64, 128, KVC_BF16, reinterpret_cast<double*>(P), P,
                           1 << 30, nullptr),
         KVC_ERR_ARG, "segment_error: ref NULL");
  expect(kvc_rank_error_curve(F, 4, 0, Fo, nullptr), KVC_ERR_ARG, "rank curve: n = 0");
  expect(kvc_rank_descriptor(P, P, 2, 2, 64, 128, KVC_BF16, 0, Fo, K32, P, 1 << 30, nullptr),
         KVC_ERR_ARG, "rank descriptor: rC = 0");
  expect(kvc_correct_rank(P, P, 2, 2, 64, 128, KVC_BF16, nullptr, F, 32, P, P, 4, 32, 0.3f,
                          nullptr, nullptr, P, P, reinterpret_cast<uint8_t*>(P), nullptr, nullptr,
                          P, 1 << 30, nullptr),
         KVC_ERR_ARG, "correct_rank: Fq NULL");
  // the error message buffer: long messages are truncated, never overrun
  char big[4096];
  std::memset(big, 'x', sizeof(big));
  big[sizeof(big) - 1] = 0;
  if (std::strlen(kvc_last_error()) >= 512) {
    std::printf("FAIL last_error longer than its buffer\n");
    ++g_fail;
  }
  std::printf(g_fail == 0 ? "abi-sanitize ok\n" : "abi-sanitize: %d failure(s)\n", g_fail);
  return g_fail == 0 ? 0 : 1;
}
