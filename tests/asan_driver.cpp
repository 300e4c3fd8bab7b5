// Host-only exercise of the C ABI for the AddressSanitizer build
// (tests/test_asan_host.py): plans of many shapes, hints, queries and every
// validation failure of the step calls, none of which reaches the GPU.  Exits
// non-zero on an unexpected status; ASan aborts on a memory error or leak.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "muon.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      std::fprintf(stderr, "line %d: %s = %d, want %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

static muon_plan_t make(const std::vector<int64_t>& m, const std::vector<int64_t>& n,
                        muon_dtype ns, muon_formulation form, int64_t cap,
                        const std::vector<muon_bucket_hint>& hints, muon_status want) {
  muon_plan_desc d{};
  muon_default_hparams(&d.hp);
  d.num_matrices = (int64_t)m.size();
  d.rows = m.data();
  d.cols = n.data();
  d.grad_dtype = MUON_BF16;
  d.ns_dtype = ns;
  d.formulation = form;
  d.max_workspace_bytes = cap;
  d.hints = hints.empty() ? nullptr : hints.data();
  d.num_hints = (int64_t)hints.size();
  muon_plan_t p = nullptr;
  size_t ws = 0;
  EXPECT(muon_plan(&d, &p, &ws), want);
  if (want != MUON_OK) return nullptr;
  int64_t nb = 0, nc = 0;
  EXPECT(muon_plan_info(p, &nb, &nc), MUON_OK);
  for (int64_t b = 0; b < nb; ++b) {
    muon_bucket_info info;
    EXPECT(muon_plan_bucket_info(p, b, &info), MUON_OK);
  }
  muon_bucket_info info;
  EXPECT(muon_plan_bucket_info(p, nb, &info), MUON_ERR_INVALID_ARGUMENT);
  size_t ws2 = 0;
  EXPECT(muon_plan_workspace_size(p, &ws2), MUON_OK);
  if (ws2 != ws) ++failures;
  return p;
}

int main() {
  std::vector<int64_t> qm, qn;  // 28 layers of Qwen2.5-7B shapes
  for (int l = 0; l < 28; ++l) {
    const int64_t s[7][2] = {{3584, 3584}, {512, 3584}, {512, 3584}, {3584, 3584},
                             {18944, 3584}, {18944, 3584}, {3584, 18944}};
    for (auto& x : s) {
      qm.push_back(x[0]);
      qn.push_back(x[1]);
    }
  }
  const std::vector<muon_bucket_hint> none;
  for (int64_t cap : {(int64_t)0, (int64_t)1, (int64_t)1 << 30}) {
    muon_plan_t p = make(qm, qn, MUON_BF16, MUON_FORM_AUTO, cap, none, MUON_OK);
    // step validation: fake pointers, nothing dereferenced or enqueued
    std::vector<float*> W(qm.size(), (float*)0x1000), M(qm.size(), (float*)0x2000);
    std::vector<const void*> G(qm.size(), (const void*)0x3000);
    size_t ws = 0;
    muon_plan_workspace_size(p, &ws);
    void* fake_ws = (void*)0x100000;
    EXPECT(muon_step_batched(p, W.data(), M.data(), G.data(), 0.02f, 0.1f, fake_ws, ws - 1, nullptr,
                             nullptr),
           MUON_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(rownorm_step(p, W.data(), M.data(), G.data(), 0.02f, 0.1f, (char*)fake_ws + 16, ws,
                        nullptr, nullptr),
           MUON_ERR_INVALID_ARGUMENT);
    G[5] = nullptr;
    EXPECT(muon_step_batched(p, W.data(), M.data(), G.data(), 0.02f, 0.1f, fake_ws, ws, nullptr,
                             nullptr),
           MUON_ERR_INVALID_ARGUMENT);
    EXPECT(muon_step_batched_noalloc(p, W.data(), M.data(), G.data(), 0.02f, 0.1f, nullptr, nullptr),
           MUON_ERR_INVALID_ARGUMENT);
    G[5] = (const void*)0x3000;
    EXPECT(muon_step_batched_noalloc(p, W.data(), M.data(), G.data(), 0.02f, 0.1f, nullptr, nullptr),
           MUON_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(muon_plan_set_profiling(p, 1), MUON_OK);
    double ms[MUON_K_COUNT];
    int64_t la[MUON_K_COUNT];
    EXPECT(muon_plan_kernel_times(p, ms, la, nullptr, nullptr), MUON_OK);
    EXPECT(muon_plan_set_profiling(p, 2), MUON_ERR_INVALID_ARGUMENT);
    EXPECT(muon_plan_destroy(p), MUON_OK);
  }
  // forms, hints and paths
  std::vector<int64_t> m = {256, 1024, 300, 64, 64, 128, 7, 1};
  std::vector<int64_t> n = {1024, 256, 300, 72, 80, 3584, 5000, 1};
  muon_plan_destroy(make(m, n, MUON_BF16, MUON_FORM_DIRECT, 0, none, MUON_OK));
  muon_plan_destroy(make(m, n, MUON_F32, MUON_FORM_GRAM, 0, none, MUON_OK));
  make(m, n, MUON_BF16, MUON_FORM_GRAM, 0, none, MUON_ERR_UNSUPPORTED);  // near-square Gram
  make(m, n, MUON_F32, MUON_FORM_DIRECT, 0, none, MUON_ERR_UNSUPPORTED);
  std::vector<muon_bucket_hint> h = {{256, 1024, 128, MUON_FORM_AUTO}, {300, 300, 64, MUON_FORM_DIRECT},
                                     {9, 9, 64, MUON_FORM_AUTO}};
  muon_plan_destroy(make(m, n, MUON_BF16, MUON_FORM_AUTO, 0, h, MUON_OK));
  h.push_back({256, 1024, 64, MUON_FORM_AUTO});  // duplicate shape
  make(m, n, MUON_BF16, MUON_FORM_AUTO, 0, h, MUON_ERR_INVALID_ARGUMENT);
  h = {{300, 300, 32, MUON_FORM_AUTO}};
  make(m, n, MUON_BF16, MUON_FORM_AUTO, 0, h, MUON_ERR_INVALID_ARGUMENT);
  // invalid descriptions
  make({}, {}, MUON_BF16, MUON_FORM_AUTO, 0, none, MUON_ERR_INVALID_ARGUMENT);
  make({0}, {5}, MUON_BF16, MUON_FORM_AUTO, 0, none, MUON_ERR_INVALID_ARGUMENT);
  make({70000}, {70000}, MUON_BF16, MUON_FORM_AUTO, 0, none, MUON_ERR_UNSUPPORTED);
  make({4}, {4}, MUON_BF16, (muon_formulation)7, 0, none, MUON_ERR_INVALID_ARGUMENT);
  EXPECT(muon_plan(nullptr, nullptr, nullptr), MUON_ERR_INVALID_ARGUMENT);
  EXPECT(muon_plan_destroy(nullptr), MUON_OK);
  for (int s = 0; s <= 5; ++s)
    if (!muon_status_string((muon_status)s)) ++failures;
  std::printf("asan driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
