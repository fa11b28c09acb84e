/* Extreme sizes through every entry point's validation (no GPU needed): each
 * call must return an error status without undefined behaviour.  Built and
 * run under AddressSanitizer and UndefinedBehaviorSanitizer (host code of
 * libmoda.so and this client), where any signed overflow, out-of-range shift
 * or invalid access in the size arithmetic aborts the run. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "moda.h"

static int failures = 0;
#define EXPECT_ERR(expr)                                                             \
  do {                                                                               \
    int got_ = (int)(expr);                                                          \
    if (got_ == MODA_OK) {                                                           \
      fprintf(stderr, "%s:%d: %s returned MODA_OK for invalid sizes\n", __FILE__,    \
              __LINE__, #expr);                                                      \
      ++failures;                                                                    \
    }                                                                                \
  } while (0)

int main(void) {
  char buf[64];
  void* F = buf; /* non-NULL, never dereferenced */
  const int M = INT_MAX, N = INT_MIN;
  const int sizes[][7] = {
      /* B, T, Hq, Hkv, d, L, dtype */
      {M, M, M, 1, 128, M, MODA_BF16}, {1, M, M, M, 128, M, MODA_BF16}, {M, 1, M, 1, 128, 1, MODA_BF16},
      {1, M, 64, 1, 128, 2, MODA_BF16}, {65536, 65536, 64, 1, 128, 48, MODA_BF16}, {N, 1, 1, 1, 128, 1, 0},
      {1, N, 1, 1, 128, 1, 1}, {1, 1, N, 1, 128, 1, 1}, {1, 1, 1, N, 128, 1, 1}, {1, 1, 1, 1, N, 1, 1},
      {1, 1, 1, 1, 128, N, 1}, {1, 1, 1, 1, M, 1, 1}, {1, 1, 1, 1, 128, 1, M}, {1, 1, 1, 1, 128, 1, N},
      {M, M, 1, 1, 64, 0, MODA_F32}, {1, 1 << 30, 1 << 20, 1, 128, 0, MODA_BF16},
  };
  const int n = (int)(sizeof(sizes) / sizeof(sizes[0]));
  long long total = 0;
  for (int i = 0; i < n; ++i) {
    const int B = sizes[i][0], T = sizes[i][1], Hq = sizes[i][2], Hkv = sizes[i][3], d = sizes[i][4];
    const int L = sizes[i][5], dt = sizes[i][6];
    total += moda_depth_packed_elems(B, T, Hkv, d, L);
    total += moda_fwd_workspace_bytes(B, T, Hq, Hkv, d, dt);
    total += moda_bwd_workspace_bytes(B, T, Hq, Hkv, d, dt);
    /* with L_d == 0 a repack has nothing to do and valid B, T succeed */
    if (L != 0) EXPECT_ERR(moda_pack_depth(F, F, F, F, B, T, Hkv, d, L, dt, NULL));
    EXPECT_ERR(moda_fwd(F, F, F, F, F, F, NULL, B, T, Hq, Hkv, d, L, dt, NULL));
    EXPECT_ERR(moda_fwd_ws(F, F, F, F, F, F, NULL, B, T, Hq, Hkv, d, L, dt, F, 256, NULL));
    EXPECT_ERR(moda_fwd_window(F, F, F, F, F, F, NULL, B, T, Hq, Hkv, d, L, 0, L, dt, NULL));
    EXPECT_ERR(moda_fwd_window(F, F, F, F, F, F, NULL, B, T, Hq, Hkv, d, L, L, N, dt, NULL));
    EXPECT_ERR(moda_append_depth(F, F, F, F, B, T, Hkv, d, L, L > N ? L - 1 : 0, dt, NULL));
    if (L != 0)
      EXPECT_ERR(moda_pack_depth_q8(F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, B, T, Hkv, d, L, dt, NULL));
    EXPECT_ERR(moda_fwd_q8(F, F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, F, NULL, B, T, Hq, Hkv, d, L,
                           dt, NULL));
    EXPECT_ERR(moda_append_depth_q8(F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, B, T, Hkv, d, L, 0, dt,
                                    NULL));
    EXPECT_ERR(moda_bwd(F, F, F, F, F, F, (const float*)F, F, F, F, F, F, F, (float*)F, B, T, Hq, Hkv, d, L, dt,
                        NULL));
    EXPECT_ERR(moda_bwd_ws(F, F, F, F, F, F, (const float*)F, F, F, F, F, F, F, B, T, Hq, Hkv, d, L, dt, F,
                           LLONG_MAX, NULL));
    EXPECT_ERR(moda_bwd_noalloc(F, F, F, F, F, F, (const float*)F, F, F, F, F, F, F, B, T, Hq, Hkv, d, L, dt,
                                NULL));
    EXPECT_ERR(moda_bwd_window_q8(F, F, F, (int8_t*)F, (int8_t*)F, (float*)F, (float*)F, F, (const float*)F, F,
                                  F, F, F, F, F, (float*)F, B, T, Hq, Hkv, d, L, 0, L, dt, NULL));
  }
  for (int s = -3; s < 10; ++s) (void)moda_status_string(s);
  (void)moda_status_string(INT_MIN);
  (void)moda_status_string(INT_MAX);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("extreme-size checks passed (%lld)\n", total);
  return 0;
}
