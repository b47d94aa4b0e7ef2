/* Host-side checks of libw12 built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on its host code (libw12_hostcheck.so). Every
 * call here returns before any HIP call: status strings, workspace sizes,
 * plans over many shapes, M, ops, flags and test hooks, and the argument
 * checks of every entry point fed fake device pointers. A sanitizer report
 * or a failed expectation exits nonzero. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "w12.h"

static int failures = 0;
#define EXPECT(c)                                                  \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, \
              __LINE__, #c);                                       \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static void* const FAKE = (void*)(uintptr_t)0x7F0000000000ull;

static w12_matrix desc(int64_t n, int64_t k, int64_t n_esc) {
  w12_matrix m;
  memset(&m, 0, sizeof m);
  m.n = n;
  m.k = k;
  m.records = (const uint8_t*)FAKE;
  m.e_top = (const uint8_t*)FAKE;
  m.esc_row_ptr = (const uint32_t*)FAKE;
  m.esc = n_esc ? (const w12_escape*)FAKE : NULL;
  m.n_esc = n_esc;
  m.format_version = W12_FORMAT_VERSION;
  return m;
}

int main(void) {
  EXPECT(w12_abi_version() == W12_ABI_VERSION);
  for (int s = -12; s <= 2; ++s) EXPECT(w12_status_str(s) != NULL && strlen(w12_status_str(s)) > 0);
  EXPECT(w12_last_error() != NULL);

  static const int64_t ns[] = {0, 16, 48, 1024, 5120, 6144, 8192, 12784, 16368, 17408, 34816, 151936, 1 << 20};
  static const int64_t ks[] = {0, 511, 512, 1024, 5120, 6144, 17408, 1 << 20, (int64_t)1 << 24};
  static const int64_t escs[] = {0, 100000};
  static const int64_t paths[] = {0, 1, 2, 3, 4, 9};
  static const int64_t grids[] = {0, 1, 7, 1000, 5000};
  size_t plans = 0;
  for (size_t pi = 0; pi < sizeof paths / sizeof *paths; ++pi) {
    for (size_t gi = 0; gi < sizeof grids / sizeof *grids; ++gi) {
      w12_set_tuning(W12_TUNE_PATH, paths[pi]);
      w12_set_tuning(W12_TUNE_GRID, grids[gi]);
      for (size_t a = 0; a < sizeof ns / sizeof *ns; ++a) {
        for (size_t b = 0; b < sizeof ks / sizeof *ks; ++b) {
          for (int op = 0; op <= 6; ++op) {
            for (int64_t M = 0; M <= 65; M += (M < 4 ? 1 : 13)) {
              const size_t ws = w12_workspace_bytes(op, ns[a], ks[b], M);
              for (size_t e = 0; e < sizeof escs / sizeof *escs; ++e) {
                const w12_matrix m = desc(ns[a], ks[b], escs[e]);
                for (uint32_t flags = 0; flags <= 2; ++flags) {
                  w12_plan p;
                  memset(&p, 0xAB, sizeof p);
                  const int r = w12_plan_info(&m, op, M, flags, &p);
                  if (r == W12_OK) {
                    ++plans;
                    EXPECT(p.grid >= 1 && p.threads >= 64);
                    EXPECT(p.workspace_bytes <= ws);
                    EXPECT(p.kernel >= W12_KERNEL_GEMV && p.kernel <= W12_KERNEL_MFMA_STREAM);
                    EXPECT(p.split_units >= 0 && p.split_tiles >= 0 && p.whole_tiles >= 0);
                  }
                }
              }
            }
          }
        }
      }
    }
  }
  w12_set_tuning(W12_TUNE_PATH, 0);
  w12_set_tuning(W12_TUNE_GRID, 0);
  EXPECT(plans > 1000);

  /* argument checks: each returns before touching the device */
  const w12_matrix m = desc(1024, 1024, 10);
  const size_t big = (size_t)1 << 40;
  EXPECT(w12_gemm(&m, FAKE, 0, 1024, FAKE, 1024, W12_F32, FAKE, big, NULL) == W12_E_M_RANGE);
  EXPECT(w12_gemm(&m, FAKE, 65, 1024, FAKE, 1024, W12_F32, FAKE, big, NULL) == W12_E_M_RANGE);
  EXPECT(w12_gemm(&m, FAKE, 4, 1000, FAKE, 1024, W12_F32, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_gemm(&m, FAKE, 4, 1024, FAKE, 1023, W12_F32, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_gemm(&m, FAKE, 4, 1024, FAKE, 1024, 7, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_gemm(&m, FAKE, 4, 1024, FAKE, 1024, W12_F32, FAKE, 16, NULL) == W12_E_WORKSPACE);
  EXPECT(w12_gemm(NULL, FAKE, 4, 1024, FAKE, 1024, W12_F32, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_gemm_q8(&m, FAKE, 4, 1024, FAKE, 1024, W12_F32, 4, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_gemm_noalloc(&m, FAKE, 0, 1024, FAKE, 1024, W12_F32, NULL) == W12_E_M_RANGE);
  EXPECT(w12_lmhead_argmax(&m, FAKE, 4, 1024, NULL, NULL, FAKE, big, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_lmhead_argmax_certified(&m, NULL, FAKE, 4, 1024, FAKE, NULL, NULL, FAKE, big, NULL) ==
         W12_E_INVALID_ARG);
  EXPECT(w12_lmhead_argmax_certified(&m, FAKE, FAKE, 4, 1024, FAKE, NULL, NULL, FAKE, 16, NULL) == W12_E_WORKSPACE);
  EXPECT(w12_certify_bounds(&m, (float*)((char*)FAKE + 4), NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_decode(&m, (uint16_t*)((char*)FAKE + 2), NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_validate(&m, NULL, 0, NULL) == W12_E_WORKSPACE);
  EXPECT(w12_encode(FAKE, 16, 512, FAKE, FAKE, FAKE, NULL, 3, NULL) == W12_E_INVALID_ARG);
  EXPECT(w12_encode(FAKE, 16, 500, FAKE, FAKE, FAKE, FAKE, 3, NULL) == W12_E_UNSUPPORTED_SHAPE);
  int64_t n_esc = 0;
  EXPECT(w12_encode_plan(FAKE, 1024, 1024, FAKE, FAKE, &n_esc, FAKE, 16, NULL) == W12_E_WORKSPACE);
  w12_matrix bad = desc(1024, 1024, 0);
  bad.format_version = 99;
  EXPECT(w12_gemm(&bad, FAKE, 4, 1024, FAKE, 1024, W12_F32, FAKE, big, NULL) == W12_E_VERSION);
  bad = desc(1024, 1024, -1);
  EXPECT(w12_plan_info(&bad, W12_OP_GEMM, 4, 0, NULL) == W12_E_INVALID_ARG);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host checks ok: %zu plans\n", plans);
  return 0;
}
