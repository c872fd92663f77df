/* Drives the C ABI's argument validation under host AddressSanitizer and
 * UndefinedBehaviorSanitizer: every call below is rejected (or is the M = 0
 * no-op) before any HIP call, so the fake device addresses are never
 * dereferenced.  Exit status 0 when every call returns the expected status. */
#include <stdint.h>
#include <stdio.h>

#include "obl.h"

#define P(a) ((void*)(uintptr_t)(a))
static int fails = 0;
static void expect(const char* what, obl_status got, obl_status want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, obl_status_string(got), (int)want);
    ++fails;
  }
}

int main(void) {
  void *X = P(0x1000000000), *W = P(0x2000000000), *A = P(0x3000000000), *B = P(0x4000000000);
  void *Y = P(0x5000000000), *WS = P(0x6000000000), *S1 = P(0x7000000000), *G = P(0x8000000000);
  const int64_t big = (int64_t)1 << 31;

  /* pack */
  expect("pack null", obl_pack_signs(NULL, OBL_I8, 4, 32, W, NULL), OBL_ERR_NULL);
  expect("pack K%32", obl_pack_signs(X, OBL_I8, 4, 33, W, NULL), OBL_ERR_SHAPE);
  expect("pack big", obl_pack_signs(X, OBL_I8, big, 32, W, NULL), OBL_ERR_SHAPE);
  expect("pack dtype", obl_pack_signs(X, (obl_dtype)9, 4, 32, W, NULL), OBL_ERR_DTYPE);
  expect("pack align", obl_pack_signs(X, OBL_I8, 4, 32, P(0x2000000002), NULL), OBL_ERR_ALIGN);
  expect("pack alias", obl_pack_signs(X, OBL_I8, 4, 32, P(0x1000000000 + 64), NULL), OBL_ERR_ALIAS);

  /* linear */
  expect("linear m0", obl_linear(NULL, OBL_BF16, 0, 4096, W, 11008, A, B, OBL_F16, NULL, OBL_F32, NULL), OBL_OK);
  expect("linear null W", obl_linear(X, OBL_BF16, 1, 4096, NULL, 11008, A, B, OBL_F16, Y, OBL_F32, NULL), OBL_ERR_NULL);
  expect("linear neg M", obl_linear(X, OBL_BF16, -1, 4096, W, 11008, A, B, OBL_F16, Y, OBL_F32, NULL), OBL_ERR_SHAPE);
  expect("linear overflow", obl_linear(X, OBL_BF16, (int64_t)1 << 40, (int64_t)1 << 30, W, 8, A, B, OBL_F16, Y,
                                       OBL_F32, NULL), OBL_ERR_SHAPE);
  expect("linear dtype", obl_linear(X, OBL_F16, 1, 4096, W, 11008, A, B, OBL_F16, Y, OBL_F32, NULL), OBL_ERR_DTYPE);
  expect("linear align", obl_linear(P(0x1000000001), OBL_BF16, 1, 4096, W, 11008, A, B, OBL_F16, Y, OBL_F32, NULL),
         OBL_ERR_ALIGN);
  expect("linear alias", obl_linear(X, OBL_BF16, 1, 4096, W, 11008, A, B, OBL_F16, P(0x1000000000 + 256), OBL_F32,
                                    NULL), OBL_ERR_ALIAS);

  /* dbf */
  expect("dbf m0", dbf_linear(NULL, OBL_BF16, 0, 4096, W, 3072, S1, 4096, B, G, A, OBL_F16, NULL, NULL, OBL_F32, NULL),
         OBL_OK);
  expect("dbf Kmid%32", dbf_linear(X, OBL_BF16, 8, 4096, W, 3000, S1, 4096, B, G, A, OBL_F16, WS, Y, OBL_F32, NULL),
         OBL_ERR_SHAPE);
  expect("dbf alias", dbf_linear(X, OBL_BF16, 8, 4096, W, 3072, S1, 4096, B, G, A, OBL_F16, P(0x5000000000 + 64), Y,
                                 OBL_F32, NULL), OBL_ERR_ALIAS);

  expect("dbf noalloc m0", dbf_linear_noalloc(NULL, OBL_BF16, 0, 4096, W, 3072, S1, 4096, B, G, A, OBL_F16, NULL,
                                             NULL, OBL_F32, NULL), OBL_OK);
  expect("dbf noalloc Kmid%32", dbf_linear_noalloc(X, OBL_BF16, 8, 4096, W, 3000, S1, 4096, B, G, A, OBL_F16, WS, Y,
                                                  OBL_F32, NULL), OBL_ERR_SHAPE);
  expect("dbf noalloc alias", dbf_linear_noalloc(X, OBL_BF16, 8, 4096, W, 3072, S1, 4096, B, G, A, OBL_F16,
                                                P(0x5000000000 + 64), Y, OBL_F32, NULL), OBL_ERR_ALIAS);

  /* svid, transpose, backward */
  expect("svid iters", obl_svid(X, OBL_F16, 64, 64, 0, W, A, B, OBL_F16, NULL), OBL_ERR_SHAPE);
  expect("svid alias", obl_svid(X, OBL_F16, 64, 64, 4, W, P(0x2000000000 + 4), B, OBL_F16, NULL), OBL_ERR_ALIAS);
  expect("transpose rows%32", obl_transpose_signs(W, 40, 64, Y, NULL), OBL_ERR_SHAPE);
  expect("backward N%32", obl_linear_backward(X, Y, OBL_BF16, 2, 64, W, S1, 40, A, B, OBL_F16, WS, OBL_F32, G,
                                              P(0x9000000000), P(0xA000000000), NULL), OBL_ERR_SHAPE);
  expect("backward alias", obl_linear_backward(X, Y, OBL_BF16, 2, 64, W, S1, 64, A, B, OBL_F16, WS, OBL_F32, G, G,
                                               P(0xA000000000), NULL), OBL_ERR_ALIAS);

  /* layernorm */
  expect("ln eps", obl_layernorm(Y, OBL_F32, 4, 64, -1.0f, NULL, NULL, OBL_F32, WS, OBL_F32, NULL), OBL_ERR_VALUE);
  expect("ln m0", obl_layernorm(NULL, OBL_F32, 0, 64, 1e-5f, NULL, NULL, OBL_F32, NULL, OBL_F32, NULL), OBL_OK);
  expect("ln alias", obl_layernorm(Y, OBL_F32, 4, 64, 1e-5f, NULL, NULL, OBL_F32, P(0x5000000000 + 16), OBL_F32,
                                   NULL), OBL_ERR_ALIAS);
  expect("lln big", obl_linear_layernorm(X, OBL_BF16, big, 32, W, 32, A, B, OBL_F16, 1e-5f, NULL, NULL, WS, Y,
                                         OBL_F32, NULL), OBL_ERR_SHAPE);

  for (int s = 0; s <= 9; ++s)
    if (!obl_status_string((obl_status)s)) ++fails;
  if (obl_version() < 100) ++fails;
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("all ABI rejection checks passed\n");
  return fails ? 1 : 0;
}
