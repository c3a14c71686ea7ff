// Drives the host-side validation of libhelmkv (include/helm_kv.h) with valid
// and invalid arguments — everything that runs before the first enqueue — for
// a build whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  No GPU is needed:
// every call here is refused, answered from host arithmetic, or stops at the
// device check.  Exit status 0 = every call returned what it should.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "helm_kv.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "%s:%d: expected %s (%s)\n", __FILE__, __LINE__, #cond, \
                   helm_last_error());                                            \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static helm_shape_t shape(int64_t T) {
  helm_shape_t s;
  std::memset(&s, 0, sizeof(s));
  s.n_src_layers = 40;
  s.n_tgt_layers = 64;
  s.n_kv_heads = 8;
  s.head_dim = 128;
  s.k = 4;
  s.dtype = HELM_BF16;
  s.n_tokens = T;
  s.rope_theta_src = 1e6;
  s.rope_theta_tgt = 1e6;
  return s;
}

int main() {
  // status names, ABI version, arch gate, last error
  for (int c = -3; c < 16; ++c) EXPECT(helm_status_string(c) != nullptr);
  EXPECT(std::strcmp(helm_status_string(HELM_OK), "HELM_OK") == 0);
  EXPECT(helm_abi_version() == HELM_ABI_VERSION);
  EXPECT(helm_arch_supported("gfx950:sramecc+:xnack-") == 1);
  EXPECT(helm_arch_supported("gfx942") == 0);
  EXPECT(helm_arch_supported("") == 0);
  EXPECT(helm_arch_supported(nullptr) == 0);
  EXPECT(helm_last_error() != nullptr);

  // workspace sizes: valid, zero tokens, invalid shapes, overflow
  helm_shape_t s = shape(32768);
  EXPECT(helm_kv_workspace_bytes(&s) > 0);
  helm_shape_t z = shape(0);
  (void)helm_kv_workspace_bytes(&z);
  helm_shape_t bad = shape(32768);
  bad.head_dim = 96;
  EXPECT(helm_kv_workspace_bytes(&bad) == 0);
  bad = shape(32768);
  bad.k = 0;
  EXPECT(helm_kv_workspace_bytes(&bad) == 0);
  bad = shape(INT64_MAX / 2);
  EXPECT(helm_kv_workspace_bytes(&bad) == 0);
  bad = shape(32768);
  bad.dtype = 7;
  EXPECT(helm_kv_workspace_bytes(&bad) == 0);
  EXPECT(helm_kv_workspace_bytes(nullptr) == 0);
  EXPECT(helm_kv_wide_workspace_bytes(&s) > 0);

  // mapper check with host layer_sel: valid, out of range, null
  std::vector<int32_t> sel(64 * 4);
  for (size_t i = 0; i < sel.size(); ++i) sel[i] = (int32_t)(i % 40);
  EXPECT(helm_mapper_check(&s, sel.data()) == HELM_OK);
  sel[17] = 40;
  EXPECT(helm_mapper_check(&s, sel.data()) == HELM_E_LAYER_SEL);
  sel[17] = -1;
  EXPECT(helm_mapper_check(&s, sel.data()) == HELM_E_LAYER_SEL);
  EXPECT(helm_mapper_check(&s, nullptr) != HELM_OK);

  // paged check: a valid batch, then broken cu_seqlens, tables and shared target slots
  helm_paged_shape_t p;
  std::memset(&p, 0, sizeof(p));
  p.n_src_layers = 28; p.n_tgt_layers = 28; p.n_kv_heads = 8; p.head_dim = 128; p.k = 4;
  p.dtype = HELM_BF16; p.block_size = 16; p.n_requests = 2; p.max_blocks_src = 3; p.max_blocks_tgt = 3;
  p.n_src_blocks = 6; p.n_tgt_blocks = 6; p.n_tokens_total = 40; p.rope_theta_src = 1e6; p.rope_theta_tgt = 1e6;
  int32_t sbt[6] = {0, 1, 2, 3, 4, -1}, tbt[6] = {5, 4, 3, 2, 1, -1}, cu[3] = {0, 33, 40};
  EXPECT(helm_paged_check(&p, sbt, tbt, cu) == HELM_OK);
  EXPECT(helm_kv_paged_workspace_bytes(&p) > 0);
  int32_t cu_bad[3] = {0, 41, 40};
  EXPECT(helm_paged_check(&p, sbt, tbt, cu_bad) == HELM_E_PAGED_TABLE);
  int32_t sbt_bad[6] = {0, 1, 9, 3, 4, -1};
  EXPECT(helm_paged_check(&p, sbt_bad, tbt, cu) == HELM_E_PAGED_TABLE);
  int32_t tbt_shared[6] = {5, 4, 3, 5, 1, -1};
  EXPECT(helm_paged_check(&p, sbt, tbt_shared, cu) == HELM_E_PAGED_TABLE);
  p.n_requests = 0;
  EXPECT(helm_paged_check(&p, sbt, tbt, cu) != HELM_OK);

  // ridge workspace: valid and refused shapes
  helm_ridge_shape_t r;
  std::memset(&r, 0, sizeof(r));
  r.n_groups = 1024; r.n_obs = 131072; r.in_features = 512; r.out_features = 128; r.dtype = HELM_BF16; r.lambda = 0.01;
  EXPECT(helm_ridge_workspace_bytes(&r) > 0);
  r.in_features = 100;
  EXPECT(helm_ridge_workspace_bytes(&r) == 0);
  r.in_features = 512;
  r.out_features = 64;
  EXPECT(helm_ridge_workspace_bytes(&r) == 0);
  r.out_features = 128;
  r.n_groups = INT64_MAX / 4;
  EXPECT(helm_ridge_workspace_bytes(&r) == 0);

  // transfers refused before any enqueue: null pointers, bad shapes, no workspace
  helm_shape_t t = shape(64);
  EXPECT(helm_kv_transfer(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, &t) != HELM_OK);
  EXPECT(helm_kv_transfer(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr) != HELM_OK);
  helm_shape_t t0 = shape(0);
  EXPECT(helm_kv_transfer(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, &t0) == HELM_OK);
  EXPECT(helm_ridge_fit(nullptr, nullptr, nullptr, nullptr, &r) != HELM_OK);

  if (failures) std::fprintf(stderr, "%d expectation(s) failed\n", failures);
  else std::printf("host checks: all calls as expected\n");
  return failures ? 1 : 0;
}
