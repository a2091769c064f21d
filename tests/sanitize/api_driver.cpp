// Host-side exercise of the C ABI for the AddressSanitizer / UndefinedBehavior
// build: plan validation (good and bad problems), size queries, algorithm and
// split-k settings, argument checks that fail before any launch, the
// multi-stream row partition's validation and the allocation-free product's
// size check. No call here reaches the device.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nmsparse.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      failures++;                                                      \
    }                                                                  \
  } while (0)

static nm_problem_t base(int64_t m, int64_t n, int64_t k, int N, int M, int dt) {
  nm_problem_t p;
  memset(&p, 0, sizeof p);
  p.m = m; p.n = n; p.k = k; p.nm_n = N; p.nm_m = M;
  p.op_a = NM_OP_N; p.op_b = NM_OP_T;
  p.type_ab = dt; p.type_cd = dt == NM_I8 ? NM_I32 : dt;
  p.lda = k; p.ldb = k; p.ldc = n; p.ldd = n;
  return p;
}

int main() {
  const int dts[3] = {NM_F16, NM_BF16, NM_I8};
  const int nms[6][2] = {{2, 4}, {1, 4}, {3, 8}, {5, 16}, {4, 32}, {8, 32}};
  // good problems of every type, N:M, layout and vector width
  for (int d = 0; d < 3; d++)
    for (int c = 0; c < 6; c++)
      for (int v = 0; v <= 64; v = v ? v * 4 : 1) {
        for (int opb = 0; opb < 2; opb++) {
          nm_problem_t p = base(256, 48 + 80 * opb, 512, nms[c][0], nms[c][1], dts[d]);
          p.op_b = opb;
          p.ldb = opb ? p.k : p.n;
          p.vector_rows = v;
          nm_plan_t plan = NULL;
          EXPECT(nm_plan_init(&plan, &p) == NM_OK);
          size_t vb = 0, mb = 0, kb = 0, ws = 0;
          int64_t vl = 0, ml = 0, kl = 0;
          EXPECT(nm_compressed_size(plan, &vb, &mb, &vl, &ml) == NM_OK);
          EXPECT(nm_mask_size(plan, &kb, &kl) == NM_OK);
          EXPECT(vb == (size_t)(256 * vl * (dts[d] == NM_I8 ? 1 : 2)));
          EXPECT(nm_plan_set_split_k(plan, 3) == NM_OK);
          EXPECT(nm_spmm_workspace_size(plan, &ws) == NM_OK);
          int32_t req = 0, eff = 0;
          EXPECT(nm_plan_get_split_k(plan, &req, &eff) == NM_OK && req == 3 && eff >= 1);
          for (int a = 0; a < nm_plan_algorithm_count(plan); a++) EXPECT(nm_plan_set_algorithm(plan, a) == NM_OK);
          EXPECT(nm_plan_set_algorithm(plan, 99) == NM_ERR_INVALID_ARG);
          EXPECT(strlen(nm_plan_kernel_name(plan)) > 0);
          // argument errors, all found before anything is enqueued
          const float one = 1.0f, zero = 0.0f;
          void* fake = (void*)0x10000;
          EXPECT(nm_spmm(plan, NULL, fake, fake, fake, &zero, NULL, fake, NULL, NULL) == NM_ERR_INVALID_ARG);
          EXPECT(nm_spmm(plan, &one, fake, (void*)0x10004, fake, &zero, NULL, fake, fake, NULL) == NM_ERR_ALIGN);
          void* streams[2] = {NULL, NULL};
          EXPECT(nm_spmm_streams(plan, &one, fake, fake, fake, &zero, NULL, fake, fake, streams, 0) ==
                 NM_ERR_INVALID_ARG);
          EXPECT(nm_prune(plan, fake, fake, 7, NULL, NULL) == NM_ERR_INVALID_ARG);
          EXPECT(nm_mask_apply(plan, NULL, fake, NULL) == NM_ERR_INVALID_ARG);
          EXPECT(nm_plan_destroy(plan) == NM_OK);
        }
      }
  // bad problems
  nm_problem_t p = base(64, 64, 130, 2, 4, NM_F16);
  nm_plan_t plan = (nm_plan_t)0x1;
  EXPECT(nm_plan_init(&plan, &p) == NM_ERR_SHAPE && plan == NULL);
  p = base(64, 64, 128, 2, 4, NM_F16); p.vector_rows = 3;
  EXPECT(nm_plan_init(&plan, &p) == NM_ERR_INVALID_ARG);
  p = base(64, 64, 128, 2, 4, NM_F16); p.vector_rows = 16; p.op_a = NM_OP_T; p.lda = 64;
  EXPECT(nm_plan_init(&plan, &p) == NM_ERR_UNSUPPORTED);
  p = base(64, 64, 128, 2, 4, NM_F16); p.lda = 132;
  EXPECT(nm_plan_init(&plan, &p) == NM_ERR_ALIGN);
  p = base((int64_t)1 << 47, 64, 128, 2, 4, NM_F16);
  EXPECT(nm_plan_init(&plan, &p) == NM_ERR_SHAPE);
  EXPECT(nm_plan_init(NULL, &p) == NM_ERR_INVALID_ARG);
  EXPECT(nm_plan_init(&plan, NULL) == NM_ERR_INVALID_ARG);
  // the allocation-free product refuses a split whose partial sums exceed its scratch
  p = base(2048, 2048, 4096, 2, 4, NM_F16);
  EXPECT(nm_plan_init(&plan, &p) == NM_OK);
  EXPECT(nm_plan_set_split_k(plan, 4) == NM_OK);
  const float one = 1.0f, zero = 0.0f;
  void* fake = (void*)0x10000;
  EXPECT(nm_spmm_noalloc(plan, &one, fake, fake, fake, &zero, NULL, fake, NULL) == NM_ERR_SHAPE);
  EXPECT(strstr(nm_last_error(), "scratch") != NULL);
  nm_plan_destroy(plan);
  for (int s = 0; s <= 5; s++) EXPECT(strncmp(nm_status_string((nm_status_t)s), "NM_", 3) == 0);
  printf("api driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
