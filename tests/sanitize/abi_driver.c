/* Drives the C ABI's host code (argument checks, shape and size arithmetic,
 * status strings) with arguments that every entry point must reject before it
 * touches a device: null and misaligned pointers, unknown dtypes, shapes at
 * and past their limits, bad temperatures and filter parameters, workspaces
 * that are too small.  spec_verify_step_workspace_size is swept over shapes
 * up to the limits (pure host arithmetic).  Built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host side by tests/test_sanitizers_cpu.py;
 * no call here launches a kernel, so no GPU is needed. */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "spec_softmax.h"

static int failures = 0;
#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    const int rc_ = (call);                                                            \
    if (rc_ != (want)) {                                                               \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_,  \
              (want));                                                                 \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

#define BAD SPEC_ERR_INVALID_ARG

int main(void) {
  /* stand-in device addresses: aligned, never dereferenced on these paths */
  void* P = (void*)(uintptr_t)0x100000;
  char* Pc = (char*)P;
  float* Pf = (float*)P;
  int32_t* Pi = (int32_t*)P;
  const float nanf_ = NAN, inff = INFINITY;

  /* spec_softmax_stats */
  EXPECT(spec_softmax_stats(NULL, P, 1, 2, 3, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, NULL, 1, 2, 3, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 7, 2, 3, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 0, 3, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 0, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, SPEC_MAX_K + 1, 100, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 0, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, SPEC_MAX_V + 1, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, 0.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, -1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, nanf_, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, inff, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, 1.0f, NULL, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 2, 3, 100, 1.0f, Pf, (float*)(Pc + 2), NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, INT_MAX, SPEC_MAX_K, SPEC_MAX_V, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(P, P, 1, 1398102, 1, 4, 1.0f, Pf, Pf, NULL), BAD);
  EXPECT(spec_softmax_stats(Pc + 1, P, 1, 2, 3, 100, 1.0f, Pf, Pf, NULL), BAD);

  /* spec_verify, spec_residual_sample, spec_verify_sample */
  EXPECT(spec_verify(P, P, 0, NULL, Pf, Pf, Pf, 2, 3, 100, 1.0f, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_verify(P, P, 0, Pi, NULL, Pf, Pf, 2, 3, 100, 1.0f, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_verify(P, P, 0, Pi, Pf, Pf, Pf, 2, 3, 100, 1.0f, NULL, Pi, NULL, NULL), BAD);
  EXPECT(spec_verify(P, P, 0, Pi, Pf, Pf, Pf, 2, 3, 100, 1.0f, Pi, Pi, (float*)(Pc + 1), NULL),
         BAD);
  EXPECT(spec_verify(P, P, 0, Pi, Pf, Pf, Pf, -5, 3, 100, 1.0f, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_residual_sample(P, P, 0, Pf, Pf, Pf, NULL, 2, 3, 100, 1.0f, Pi, NULL, NULL), BAD);
  EXPECT(spec_residual_sample(P, P, 0, Pf, Pf, Pf, Pi, 2, 3, 100, 1.0f, Pi, (int32_t*)(Pc + 1),
                              NULL),
         BAD);
  EXPECT(spec_residual_sample(P, P, 0, Pf, Pf, Pf, Pi, 2, 3, 100, nanf_, Pi, NULL, NULL), BAD);
  EXPECT(spec_verify_sample(P, P, 1, Pi, Pf, Pf, Pf, 1398102, 1, 4, 1.0f, Pi, Pi, NULL, NULL,
                            NULL),
         BAD);
  EXPECT(spec_verify_sample(P, P, 1, Pi, Pf, NULL, Pf, 2, 3, 100, 1.0f, Pi, Pi, NULL, NULL, NULL),
         BAD);
  EXPECT(spec_verify_sample(P, P, 1, Pi, Pf, Pf, Pf, 2, 3, 100, 1.0f, Pi, NULL, NULL, NULL, NULL),
         BAD);

  /* spec_greedy_verify, spec_sample, spec_filter */
  EXPECT(spec_greedy_verify(P, 5, Pi, 2, 3, 100, Pi, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_greedy_verify(P, 1, NULL, 2, 3, 100, Pi, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_greedy_verify(P, 1, Pi, 2, 0, 100, Pi, Pi, Pi, NULL, NULL), BAD);
  EXPECT(spec_greedy_verify(P, 1, Pi, 2, 3, 100, Pi, Pi, Pi, (int32_t*)(Pc + 2), NULL), BAD);
  EXPECT(spec_sample(NULL, 1, 4, 100, 1.0f, Pf, Pf, Pi, NULL), BAD);
  EXPECT(spec_sample(P, 1, 0, 100, 1.0f, Pf, Pf, Pi, NULL), BAD);
  EXPECT(spec_sample(P, 1, 4194304, 4, 1.0f, Pf, Pf, Pi, NULL), BAD);
  EXPECT(spec_sample(P, 1, 4, 100, -2.0f, Pf, Pf, Pi, NULL), BAD);
  EXPECT(spec_sample(P, 1, 4, 100, 1.0f, Pf, Pf, (int32_t*)(Pc + 1), NULL), BAD);
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, -1, 0.9f, Pf, NULL, NULL, NULL), BAD);
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, 2, 0.0f, Pf, NULL, NULL, NULL), BAD);
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, 2, nanf_, Pf, NULL, NULL, NULL), BAD);
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, 2, 0.9f, NULL, NULL, NULL, NULL), BAD);
  EXPECT(spec_filter(P, 1, 4194304, 4, 1.0f, 2, 1.0f, Pf, NULL, NULL, NULL), BAD);
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, 2, 0.9f, Pf, NULL, Pc + 100, NULL), BAD); /* overlap */
  EXPECT(spec_filter(P, 1, 4, 100, 1.0f, 2, 0.9f, Pf, (float*)(Pc + 2), NULL, NULL), BAD);

  /* spec_verify_step and its no-allocation variant */
  const size_t need = spec_verify_step_workspace_size(2, 3, 100, 1);
  if (need == 0) {
    fprintf(stderr, "workspace size of a valid shape is 0\n");
    ++failures;
  }
  EXPECT(spec_verify_step(P, P, 1, Pi, Pf, 2, 3, 100, 1.0f, Pf, Pf, Pi, Pi, NULL, NULL, NULL, need,
                          NULL),
         BAD);
  EXPECT(spec_verify_step(P, P, 1, Pi, Pf, 2, 3, 100, 1.0f, Pf, Pf, Pi, Pi, NULL, NULL, P,
                          need - 1, NULL),
         BAD);
  EXPECT(spec_verify_step(P, P, 1, Pi, Pf, 2, 3, 100, 1.0f, Pf, Pf, Pi, Pi, NULL, NULL, Pc + 16,
                          need, NULL),
         BAD);
  EXPECT(spec_verify_step(P, P, 1, Pi, Pf, 2, 3, 100, -1.0f, Pf, Pf, Pi, Pi, NULL, NULL, P, need,
                          NULL),
         BAD);
  EXPECT(spec_verify_step_noalloc(P, P, 1, NULL, Pf, 2, 3, 100, 1.0f, Pf, Pf, Pi, Pi, NULL, NULL,
                                  NULL),
         BAD);
  EXPECT(spec_verify_step_noalloc(P, P, 0, Pi, Pf, 31, 1, 1 << 20, 1.0f, Pf, Pf, Pi, Pi, NULL,
                                  NULL, NULL),
         SPEC_ERR_UNSUPPORTED);

  /* the workspace arithmetic over shapes up to the limits, and past them */
  const int Bs[] = {1, 2, 31, 64, 65, 1000, 4194303 / 129, 4194303 / 3, 4194303, INT_MAX};
  const int Ks[] = {1, 2, 8, 63, 64, 65};
  const int Vs[] = {1, 7, 1024, 32000, 128256, SPEC_MAX_V, SPEC_MAX_V + 1};
  size_t prev = 0;
  for (size_t b = 0; b < sizeof Bs / sizeof Bs[0]; ++b)
    for (size_t k = 0; k < sizeof Ks / sizeof Ks[0]; ++k)
      for (size_t v = 0; v < sizeof Vs / sizeof Vs[0]; ++v)
        for (int dt = -1; dt <= 2; ++dt) {
          const size_t n = spec_verify_step_workspace_size(Bs[b], Ks[k], Vs[v], dt);
          const int valid = Ks[k] <= SPEC_MAX_K && Vs[v] <= SPEC_MAX_V && (dt == 0 || dt == 1) &&
                            (int64_t)Bs[b] * (2 * Ks[k] + 1) <= SPEC_MAX_ROWS;
          if (valid != (n != 0)) {
            fprintf(stderr, "workspace size %zu for B=%d K=%d V=%d dtype=%d\n", n, Bs[b], Ks[k],
                    Vs[v], dt);
            ++failures;
          }
          prev += n;
        }

  /* status strings: every code, and some that are none */
  for (int c = -3; c <= 8; ++c) {
    const char* s = spec_status_string(c);
    if (s == NULL || strlen(s) == 0) {
      fprintf(stderr, "no status string for %d\n", c);
      ++failures;
    }
  }
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi driver: ok (%zu workspace bytes summed)\n", prev);
  return 0;
}
