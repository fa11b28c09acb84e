/* Plain C client of libmoda.so: the header compiles as C, every entry point
 * links, and argument validation returns the documented codes before any HIP
 * call (so this runs without a GPU).  Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moda.h"

static int failures = 0;
#define EXPECT(expr, want)                                                         \
  do {                                                                             \
    int got_ = (int)(expr);                                                        \
    if (got_ != (want)) {                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, \
              #expr, got_, (int)(want));                                           \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

int main(void) {
  char buf[64];
  void* F = buf; /* a non-NULL pointer that is never dereferenced */

  EXPECT(moda_depth_packed_elems(1, 77, 3, 128, 5) == 3LL * 416 * 128, 1);
  EXPECT(moda_depth_packed_elems(1, 5, 1, 64, 0), 0);
  EXPECT(moda_depth_packed_elems(0, 5, 1, 64, 1), -1);

  EXPECT(moda_pack_depth(NULL, NULL, NULL, NULL, 1, 4, 1, 128, 0, MODA_BF16, NULL), MODA_OK);
  EXPECT(moda_pack_depth(NULL, F, F, F, 1, 4, 1, 128, 2, MODA_BF16, NULL), MODA_ERR_NULL);
  EXPECT(moda_pack_depth(F, F, F, F, 1, 4, 1, 96, 2, MODA_BF16, NULL), MODA_ERR_UNSUPPORTED);

  EXPECT(moda_fwd(F, F, F, NULL, NULL, F, NULL, 1, 4, 3, 2, 128, 0, MODA_BF16, NULL), MODA_ERR_SHAPE);
  EXPECT(moda_fwd(F, F, F, NULL, NULL, F, NULL, 1, 4, 2, 1, 128, 0, 7, NULL), MODA_ERR_DTYPE);
  EXPECT(moda_fwd(F, F, F, NULL, F, F, NULL, 1, 4, 2, 1, 128, 3, MODA_BF16, NULL), MODA_ERR_NULL);
  EXPECT(moda_fwd_window(F, F, F, F, F, F, NULL, 1, 4, 2, 1, 128, 4, 0, 5, MODA_BF16, NULL), MODA_ERR_SHAPE);
  EXPECT(moda_append_depth(F, F, F, F, 1, 4, 1, 128, 3, 3, MODA_BF16, NULL), MODA_ERR_SHAPE);
  EXPECT(moda_bwd_noalloc(F, F, F, NULL, NULL, F, (const float*)F, F, F, F, F, NULL, NULL, 1, 65537, 64, 1, 128,
                          0, MODA_BF16, NULL),
         MODA_ERR_WORKSPACE);
  EXPECT(moda_bwd_workspace_bytes(1, 4096, 16, 2, 128, MODA_BF16) > 2LL * 16 * 4096 * 4, 1);
  EXPECT(moda_bwd_workspace_bytes(1, 4096, 16, 2, 128, MODA_F32), 2LL * 16 * 4096 * 4);
  EXPECT(moda_bwd_ws(F, F, F, NULL, NULL, F, (const float*)F, F, F, F, F, NULL, NULL, 1, 4096, 16, 2, 128, 0,
                     MODA_BF16, NULL, 1 << 30, NULL),
         MODA_ERR_WORKSPACE);
  EXPECT(moda_fwd_workspace_bytes(1, 4096, 16, 2, 128, MODA_BF16) > 0, 1);
  EXPECT(moda_fwd_workspace_bytes(1, 4096, 16, 2, 128, MODA_F32), 0);
  EXPECT(moda_fwd_ws(F, F, F, F, F, F, NULL, 1, 4096, 16, 2, 128, 24, MODA_BF16, NULL, 1 << 30, NULL),
         MODA_ERR_WORKSPACE);

  EXPECT(moda_pack_depth_q8(F, F, (int8_t*)F, (int8_t*)F, NULL, (float*)F, 1, 4, 1, 128, 3, MODA_BF16, NULL),
         MODA_ERR_NULL);
  EXPECT(moda_fwd_q8(F, F, F, (int8_t*)F, (int8_t*)F, NULL, (float*)F, F, NULL, 1, 4, 2, 1, 128, 3, MODA_BF16,
                     NULL),
         MODA_ERR_NULL);
  EXPECT(moda_fwd_window_q8(F, F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, F, NULL, 1, 4, 2, 1, 128, 4,
                            3, 2, MODA_BF16, NULL),
         MODA_ERR_SHAPE);
  EXPECT(moda_append_depth_q8(F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, 1, 4, 1, 128, 3, -1,
                              MODA_BF16, NULL),
         MODA_ERR_SHAPE);

  EXPECT(moda_bwd(F, F, F, F, F, F, (const float*)F, F, F, F, F, F, F, NULL, 1, 4, 2, 1, 128, 3, MODA_BF16, NULL),
         MODA_ERR_NULL);
  EXPECT(moda_bwd_window(F, F, F, F, F, F, (const float*)F, F, F, F, F, F, F, (float*)F, 1, 4, 2, 1, 128, 4, 3,
                         2, MODA_BF16, NULL),
         MODA_ERR_SHAPE);

  EXPECT(moda_bwd_q8(F, F, F, (int8_t*)F, (int8_t*)F, NULL, (float*)F, F, (const float*)F, F, F, F, F, F, F,
                     (float*)F, 1, 4, 2, 1, 128, 3, MODA_BF16, NULL),
         MODA_ERR_NULL);
  EXPECT(moda_bwd_window_q8(F, F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, F, (const float*)F, F, F, F,
                            F, F, F, (float*)F, 1, 4, 2, 1, 128, 4, 3, 2, MODA_BF16, NULL),
         MODA_ERR_SHAPE);

  EXPECT(strcmp(moda_status_string(MODA_OK), "MODA_OK"), 0);
  EXPECT(strncmp(moda_status_string(MODA_ERR_NULL), "MODA_ERR_NULL", 13), 0);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("C ABI checks passed\n");
  return 0;
}
