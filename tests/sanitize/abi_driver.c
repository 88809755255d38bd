/* Argument and size checks of the C ABI (include/flashmask.h), for a host
 * build of the ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Every call here must be turned away by the checks (or be a pure query):
 * the pointers are made-up aligned addresses, so a call that got as far as a
 * launch would hand them to the GPU. Each call states the status it must
 * return; the program prints one line per call and exits nonzero on any
 * mismatch. It never runs where a GPU is present. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flashmask.h"

static int failures = 0;

#define EXPECT(expr, want)                                                   \
  do {                                                                       \
    const long long got_ = (long long)(expr);                                \
    if (got_ != (long long)(want)) {                                         \
      printf("FAIL %s: got %lld want %lld\n", #expr, got_, (long long)(want)); \
      ++failures;                                                            \
    } else {                                                                 \
      printf("ok %s\n", #expr);                                              \
    }                                                                        \
  } while (0)

#define P(x) ((void*)(uintptr_t)(x))
#define PI(x) ((int32_t*)(uintptr_t)(x))
#define PF(x) ((float*)(uintptr_t)(x))
#define A 0x100000   /* an aligned made-up address */
#define MIS 0x100001 /* a misaligned one */

enum { OK = FM_SUCCESS, INV = FM_ERROR_INVALID_VALUE, NS = FM_ERROR_NOT_SUPPORTED,
       WS = FM_ERROR_WORKSPACE_TOO_SMALL };

/* forward with one argument varied from a valid call */
static fm_status_t fwd(void* q, void* o, float* lse, int B, int H, int N, int d, int dv, int dtype,
                       int hm, int causal, const int32_t* uts, const int32_t* ute, void* ws,
                       size_t ws_bytes) {
  return flashmask_fwd(q, P(A), P(A), PI(A), NULL, uts, ute, hm, NULL, B, H, N, d, dv,
                       (fm_dtype_t)dtype, causal, 0.f, o, lse, NULL, ws, ws_bytes, NULL);
}

static fm_status_t bwd(void* q, void* dq, int B, int H, int N, int d, int dv, int dtype, void* ws,
                       size_t ws_bytes) {
  return flashmask_bwd(q, P(A), P(A), P(A), PF(A), P(A), PI(A), NULL, NULL, NULL, 1, NULL, B, H, N,
                       d, dv, (fm_dtype_t)dtype, 1, 0.f, dq, P(A), P(A), NULL, ws, ws_bytes, NULL);
}

int main(void) {
  /* pure queries */
  for (int s = -2; s < 8; ++s) EXPECT(strlen(flashmask_status_string((fm_status_t)s)) > 0, 1);
  EXPECT(flashmask_table_block() > 0, 1);
  EXPECT(flashmask_max_chunks() > 0, 1);
  int bq = 0, bk = 0;
  EXPECT(flashmask_tile_shape(0, 128, FM_BF16, &bq, &bk), OK);
  EXPECT(flashmask_tile_shape(1, 512, FM_BF16, &bq, &bk), OK);
  EXPECT(flashmask_tile_shape(1, 96, FM_BF16, &bq, &bk), NS);
  EXPECT(flashmask_tile_shape(1, 128, FM_BF16, NULL, &bk), INV);
  EXPECT(flashmask_tile_shape(1, 128, (fm_dtype_t)9, &bq, &bk), NS);

  /* workspace sizes: valid, invalid, and sizes too large to address */
  EXPECT(flashmask_workspace_size(0, 1, 32, 8192, 128, 128, 1, FM_BF16) > 0, 1);
  EXPECT(flashmask_workspace_size(1, 1, 32, 8192, 128, 128, 1, FM_BF16) > 0, 1);
  EXPECT(flashmask_workspace_size(1, -1, 32, 8192, 128, 128, 1, FM_BF16), 0);
  EXPECT(flashmask_workspace_size(1, 1, 32, 8192, 96, 96, 1, FM_BF16), 0);
  EXPECT(flashmask_workspace_size(1, 1, 32, 8192, 128, 128, 0, FM_BF16), 0);
  EXPECT(flashmask_workspace_size(1, INT_MAX, INT_MAX, 1 << 20, 128, 128, 1, FM_BF16), 0);
  EXPECT(flashmask_workspace_size(1, INT_MAX, INT_MAX, INT_MAX, 64, 64, INT_MAX, FM_BF16), 0);
  EXPECT(flashmask_workspace_size_qk(1, INT_MAX, 1, INT_MAX, INT_MAX, 64, 64, 1, FM_FP32), 0);

  /* forward */
  EXPECT(fwd(NULL, P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), NULL, PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), NULL, 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(MIS), P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(MIS), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 96, 96, 1, 1, 1, NULL, NULL, P(A), 1 << 20), NS);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 64, 1, 1, 1, NULL, NULL, P(A), 1 << 20), NS);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 512, 512, 0, 1, 1, NULL, NULL, P(A), 1 << 20), NS);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 128, 7, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), -1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), 1, -2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, -300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 4, 300, 128, 128, 1, 3, 1, NULL, NULL, P(A), 1 << 20), INV);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 4, 300, 128, 128, 1, 0, 1, NULL, NULL, P(A), 1 << 20), INV);
  /* non-causal with one of the upper vectors missing */
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 0, PI(A), NULL, P(A), 1 << 20), INV);
  /* rows too long for 32-bit offsets, too many rows in all */
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, INT_MAX, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), NS);
  EXPECT(fwd(P(A), P(A), PF(A), INT_MAX, INT_MAX, 1 << 20, 128, 128, 1, 1, 1, NULL, NULL, P(A), 1 << 20), NS);
  EXPECT(fwd(P(A), P(A), PF(A), INT_MAX, INT_MAX, 1 << 20, 64, 64, 0, INT_MAX, 1, NULL, NULL, P(A), 1 << 20), NS);
  /* workspace missing, too small, misaligned */
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, NULL, 0), WS);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A), 16), WS);
  EXPECT(fwd(P(A), P(A), PF(A), 1, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, P(A + 16), 1 << 20), INV);
  /* empty problems are successful no-ops before any pointer is looked at */
  EXPECT(fwd(NULL, NULL, NULL, 0, 2, 300, 128, 128, 1, 1, 1, NULL, NULL, NULL, 0), OK);
  EXPECT(fwd(NULL, NULL, NULL, 1, 2, 0, 128, 128, 1, 1, 1, NULL, NULL, NULL, 0), OK);

  /* backward */
  EXPECT(bwd(NULL, P(A), 1, 2, 300, 128, 128, 1, P(A), 1 << 22), INV);
  EXPECT(bwd(P(A), NULL, 1, 2, 300, 128, 128, 1, P(A), 1 << 22), INV);
  EXPECT(bwd(P(MIS), P(A), 1, 2, 300, 128, 128, 1, P(A), 1 << 22), INV);
  EXPECT(bwd(P(A), P(A), 1, 2, 300, 80, 80, 1, P(A), 1 << 22), NS);
  EXPECT(bwd(P(A), P(A), 1, 2, 300, 128, 128, 1, P(A), 64), WS);
  EXPECT(bwd(P(A), P(A), 1, 2, 300, 128, 128, 1, NULL, 1 << 22), WS);
  EXPECT(bwd(P(A), P(A), INT_MAX, INT_MAX, 1 << 20, 128, 128, 1, P(A), 1 << 22), NS);
  EXPECT(flashmask_bwd_noalloc(P(A), P(A), P(A), P(A), PF(A), P(A), PI(A), NULL, NULL, NULL, 1, NULL,
                               64, 64, 4096, 4096, 128, 128, FM_BF16, 1, 0.f, NULL, P(A), P(A), P(A),
                               NULL, NULL, NULL),
         WS);
  EXPECT(flashmask_bwd_noalloc(NULL, P(A), P(A), P(A), PF(A), P(A), PI(A), NULL, NULL, NULL, 1, NULL,
                               1, 2, 300, 300, 96, 96, FM_BF16, 1, 0.f, NULL, P(A), P(A), P(A), NULL,
                               NULL, NULL),
         NS);

  /* tile classification and localisation */
  EXPECT(flashmask_tile_classify(PI(A), NULL, NULL, NULL, 1, 1, 300, 1, 128, 64, NULL, NULL, NULL), INV);
  EXPECT(flashmask_tile_classify(PI(A), NULL, NULL, NULL, 1, 1, 300, 1, 128, 64, PI(MIS), NULL, NULL), INV);
  EXPECT(flashmask_tile_classify(PI(A), NULL, NULL, NULL, 1, 1, 300, 1, 0, 64, PI(A), NULL, NULL), INV);
  EXPECT(flashmask_tile_classify(PI(A), NULL, NULL, NULL, -1, 1, 300, 1, 128, 64, PI(A), NULL, NULL), INV);
  EXPECT(flashmask_tile_classify(PI(A), NULL, PI(A), NULL, 1, 1, 300, 0, 128, 64, PI(A), NULL, NULL), INV);
  EXPECT(flashmask_tile_classify(NULL, NULL, NULL, NULL, 0, 1, 300, 1, 128, 64, NULL, NULL, NULL), OK);
  const int32_t good[4] = {0, 100, 200, 300};
  const int32_t overlap[4] = {0, 200, 100, 300};
  const int32_t empty[2] = {50, 50};
  const int32_t outside[2] = {0, 301};
  int32_t* o4 = PI(A);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, NULL, 1, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, good, 0, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, good, flashmask_max_chunks() + 1,
                            o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, overlap, 2, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, empty, 1, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, outside, 1, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 1, 300, 300, 1, good, 2, NULL, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(PI(A), NULL, NULL, NULL, 1, 0, 300, 300, 1, good, 2, o4, o4, o4, o4, NULL), INV);
  EXPECT(flashmask_localize(NULL, NULL, NULL, NULL, 0, 1, 300, 300, 1, good, 2, NULL, NULL, NULL, NULL, NULL), OK);

  printf("%d failure(s)\n", failures);
  return failures != 0;
}
