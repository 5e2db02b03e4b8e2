/* The C ABI used from plain C99 (no Python, no torch in the process): the
 * header compiles as C, the library links and loads, and the host-side
 * parts answer without a GPU -- version, status text, workspace queries and
 * argument validation, whose errors return before any HIP call. Calls that
 * would pass validation are never made here (they would launch kernels).
 * Exit status 0 and a final "ok" line on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gla.h"

static int failures = 0;

#define EXPECT(cond)                                                    \
  do {                                                                  \
    if (!(cond)) {                                                      \
      printf("FAILED line %d: %s\n", __LINE__, #cond);                  \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

int main(void) {
  /* stand-in device addresses: 16-byte aligned, 1 TiB apart so that no
     two ranges overlap, never dereferenced (every call below fails
     validation first) */
  void *const A = (void *)((uintptr_t)1 << 40);
  void *const B = (void *)((uintptr_t)2 << 40);
  void *const C = (void *)((uintptr_t)3 << 40);
  void *const O = (void *)((uintptr_t)4 << 40);
  const float lam[16] = {0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f,
                         0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f};
  float bad_lam[16];
  int s;

  EXPECT(gla_abi_version() == GLA_ABI_VERSION);
  for (s = GLA_OK; s <= GLA_ERR_TOO_LARGE; ++s) {
    const char *t = gla_status_str((gla_status)s);
    EXPECT(t != NULL && strlen(t) > 0);
  }

  /* the Laplace prefill shape runs as one kernel without scratch; one long
     sequence needs time segments and their states */
  EXPECT(gla_chunk_fwd_workspace_bytes(GLA_BF16, 8, 2048, 16, 96, 192, 64) == 0);
  EXPECT(gla_chunk_fwd_workspace_bytes(GLA_BF16, 1, 65536, 16, 96, 192, 64) > 0);
  /* the backward of the Laplace batch runs both walks in one launch (no
     scratch); one long sequence needs time segments */
  EXPECT(gla_chunk_bwd_workspace_bytes(GLA_BF16, 8, 2048, 16, 96, 192, 64) == 0);
  EXPECT(gla_chunk_bwd_workspace_bytes(GLA_BF16, 1, 65536, 16, 96, 192, 64) > 0);
  EXPECT(gla_chunk_fwd_varlen_workspace_bytes(GLA_BF16, 32, 120891, 16, 96, 192, 0) > 0);

  /* validation errors, each returned before any HIP call */
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 64, 16, 96, 192, 0, NULL, B, C, lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_NULL);
  EXPECT(gla_chunk_fwd((gla_dtype)7, 1, 64, 16, 96, 192, 0, A, B, C, lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_DTYPE);
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 64, 16, 100, 192, 0, A, B, C, lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_UNSUPPORTED);
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, -1, 16, 96, 192, 0, A, B, C, lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_SHAPE);
  memcpy(bad_lam, lam, sizeof(lam));
  bad_lam[3] = 0.0f;
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 64, 16, 96, 192, 0, A, B, C, bad_lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_DECAY);
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 64, 16, 96, 192, 0, A, B, C, lam, 1.0f, NULL, A,
                       NULL, NULL, 0, NULL) == GLA_ERR_ALIAS);
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 64, 16, 96, 192, 0, (char *)A + 2, B, C, lam, 1.0f,
                       NULL, O, NULL, NULL, 0, NULL) == GLA_ERR_ALIGN);
  /* a shape that needs scratch, called without it */
  EXPECT(gla_chunk_fwd(GLA_BF16, 1, 65536, 16, 96, 192, 0, A, B, C, lam, 1.0f, NULL, O,
                       NULL, NULL, 0, NULL) == GLA_ERR_WORKSPACE);
  EXPECT(gla_decode_step(GLA_BF16, 4, 16, 96, 192, A, B, C, lam, 1.0f, NULL, O, NULL) ==
         GLA_ERR_NULL);
  EXPECT(gla_decode_step_pool(GLA_BF16, 4, 16, 96, 192, A, B, C, lam, 1.0f, NULL, 8,
                              (float *)O, (char *)O + 4096 * 1024, NULL) == GLA_ERR_NULL);
  /* the allocation-free packed forward validates the same way, and refuses a
     chunk it does not run */
  EXPECT(gla_chunk_fwd_varlen_noalloc(GLA_BF16, 2, 128, 16, 96, 192, 0, NULL, A, B, C, lam,
                                      1.0f, NULL, O, NULL, NULL) == GLA_ERR_NULL);
  EXPECT(gla_chunk_fwd_varlen_noalloc(GLA_BF16, 2, 128, 16, 96, 192, 128, (int32_t *)O, A, B,
                                      C, lam, 1.0f, NULL, (char *)O + 4096, NULL,
                                      NULL) == GLA_ERR_UNSUPPORTED);
  EXPECT(gla_chunk_fwd_varlen_noalloc(GLA_BF16, 0, 128, 16, 96, 192, 0, (int32_t *)O, A, B, C,
                                      lam, 1.0f, NULL, (char *)O + 4096, NULL,
                                      NULL) == GLA_ERR_SHAPE);
  /* empty batches are valid and do nothing */
  EXPECT(gla_decode_step(GLA_BF16, 0, 16, 96, 192, A, B, C, lam, 1.0f, (float *)O, A, NULL) ==
         GLA_OK);

  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
