/* Host-side argument checks of libmoe_ep.so, driven from plain C.
 *
 * Every call below is rejected (or has nothing to launch) before the library
 * makes any HIP call, so the program needs no GPU.  The size helpers are also
 * fed extreme shapes, where their arithmetic could overflow.  tests/test_abi_sanitized.py
 * builds the library's host code and this program with AddressSanitizer and
 * UndefinedBehaviorSanitizer and runs it: any out-of-bounds access, signed
 * overflow or invalid shift in those paths fails the run.
 *
 * Pointers are fake, suitably aligned addresses: the checks look only at
 * nullness and alignment and never dereference them.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_ep.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                   \
  do {                                                                                       \
    const int got_ = (int)(expr);                                                            \
    if (got_ != (int)(want)) {                                                               \
      fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #expr, got_, (int)(want)); \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

#define A ((void*)(uintptr_t)0x100000)             /* 256-byte aligned */
#define A2 ((void*)((uintptr_t)0x100000 + 2))      /* misaligned for everything but bytes */

static moe_shape shape(int32_t T, int32_t H, int32_t k, int32_t E, int32_t R) {
  moe_shape s;
  s.num_tokens = T;
  s.hidden = H;
  s.num_topk = k;
  s.num_experts = E;
  s.num_ranks = R;
  return s;
}

static moe_status layout(const moe_shape* s, void* topk, void* ws, size_t ws_bytes) {
  return moe_get_dispatch_layout(s, topk, A, A, A, ws, ws_bytes, NULL);
}

static moe_status dispatch(const moe_shape* s, int dtype, void* x, int32_t cap, size_t ws_bytes, void* scales) {
  return moe_dispatch(s, (moe_dtype)dtype, x, A, A, A, ws_bytes, cap, A, scales, A, A, A, A, A, A, NULL);
}

static moe_status combine(const moe_shape* s, void* y, int32_t rows, void* out) {
  return moe_combine(s, y, rows, A, A, A, out, NULL);
}

int main(void) {
  const size_t big = (size_t)1 << 40;

  /* status strings */
  if (!moe_status_string(MOE_OK) || !moe_status_string((moe_status)99)) ++failures;

  /* size helpers, ordinary and extreme shapes */
  {
    moe_shape s = shape(4096, 7168, 8, 256, 8);
    EXPECT(moe_max_recv_rows(&s), 4096 * 8);
    if (moe_workspace_bytes(&s) == 0 || moe_ll_workspace_bytes(&s) == 0) ++failures;
    const int32_t extremes[][5] = {
        {INT32_MAX, 7168, 32, 4096, 64}, {INT32_MAX, INT32_MAX - 7, 32, 4096, 64},
        {INT32_MAX, 8, 1, 1, 1},         {1, INT32_MAX, 1, 1, 1},
        {-1, 8, 1, 1, 1},                {INT32_MIN, 8, 1, 1, 1},
        {16, 8, INT32_MAX, 4096, 64},    {16, 8, 8, INT32_MAX, 1},
        {16, 8, 8, 64, INT32_MAX},       {16, 8, 8, INT32_MIN, INT32_MIN},
        {0, 0, 0, 0, 0},
    };
    for (size_t i = 0; i < sizeof(extremes) / sizeof(extremes[0]); ++i) {
      moe_shape e = shape(extremes[i][0], extremes[i][1], extremes[i][2], extremes[i][3], extremes[i][4]);
      (void)moe_max_recv_rows(&e);
      (void)moe_workspace_bytes(&e);
      (void)moe_ll_workspace_bytes(&e);
      /* too large or invalid: rejected before any launch */
      if (layout(&e, A, A, big) == MOE_OK && e.num_tokens != 0) ++failures;
      if (combine(&e, A, 1, A) == MOE_OK && e.num_tokens != 0) ++failures;
    }
    EXPECT(moe_max_recv_rows(NULL), -1);
    EXPECT(moe_workspace_bytes(NULL), 0);
  }

  /* shape errors, for every entry point taking a shape */
  {
    const int32_t bad[][6] = {
        /* T, H, k, E, R, expected */
        {-1, 256, 4, 16, 4, MOE_ERR_INVALID_ARG}, {64, 0, 4, 16, 4, MOE_ERR_INVALID_ARG},
        {64, 12, 4, 16, 4, MOE_ERR_INVALID_ARG},  {64, 256, 0, 16, 4, MOE_ERR_INVALID_ARG},
        {64, 256, 4, 0, 4, MOE_ERR_INVALID_ARG},  {64, 256, 4, 16, 0, MOE_ERR_INVALID_ARG},
        {64, 256, 4, 16, 3, MOE_ERR_INVALID_ARG}, {64, 256, 4, 4, 8, MOE_ERR_INVALID_ARG},
        {64, 256, 5, 4, 4, MOE_ERR_INVALID_ARG},  {64, 256, 33, 64, 4, MOE_ERR_UNSUPPORTED},
        {64, 256, 4, 256, 128, MOE_ERR_UNSUPPORTED}, {64, 256, 4, 8192, 8, MOE_ERR_UNSUPPORTED},
    };
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
      moe_shape s = shape(bad[i][0], bad[i][1], bad[i][2], bad[i][3], bad[i][4]);
      const int want = bad[i][5];
      moe_router r = {MOE_GATE_SOFTMAX, 1, 1};
      EXPECT(layout(&s, A, A, big), want);
      EXPECT(dispatch(&s, MOE_BF16, A, 1 << 20, big, A), want);
      EXPECT(combine(&s, A, 1, A), want);
      EXPECT(moe_dispatch_ll(&s, MOE_BF16, A, A, A, big, 1 << 20, A, A, A, A, A, NULL), want);
      EXPECT(moe_combine_ll(&s, A, 1 << 20, A, A, A, A, NULL), want);
      EXPECT(moe_combine_backward(&s, A, A, 1, A, A, A, A, A, NULL), want);
      EXPECT(moe_dispatch_backward(&s, A, 1, A, A, A, A, A, NULL), want);
      EXPECT(moe_layout_dispatch(&s, MOE_BF16, A, A, A, A, A, A, A, big, 1 << 20, A, A, A, A, A, A, A, A, NULL),
             want);
      if (want == MOE_ERR_INVALID_ARG) EXPECT(moe_route_layout(&s, &r, A, A, A, A, A, A, A, big, NULL), want);
    }
  }

  /* argument errors */
  {
    moe_shape s = shape(64, 256, 4, 16, 4);
    const size_t need = moe_workspace_bytes(&s);
    EXPECT(layout(NULL, A, A, big), MOE_ERR_INVALID_ARG);
    EXPECT(layout(&s, NULL, A, big), MOE_ERR_INVALID_ARG);
    EXPECT(layout(&s, A2, A, big), MOE_ERR_INVALID_ARG);
    EXPECT(layout(&s, A, (char*)A + 16, big), MOE_ERR_INVALID_ARG);
    EXPECT(layout(&s, A, A, need - 1), MOE_ERR_INVALID_ARG);

    EXPECT(dispatch(&s, 2, A, 256, big, A), MOE_ERR_INVALID_ARG);
    EXPECT(dispatch(&s, MOE_BF16, A, 255, big, A), MOE_ERR_CAPACITY);
    EXPECT(dispatch(&s, MOE_BF16, A, -1, big, A), MOE_ERR_INVALID_ARG);
    EXPECT(dispatch(&s, MOE_BF16, (char*)A + 8, 256, big, A), MOE_ERR_INVALID_ARG);
    EXPECT(dispatch(&s, MOE_BF16, A, 256, 16, A), MOE_ERR_INVALID_ARG);
    EXPECT(dispatch(&s, MOE_FP8_E4M3, A, 256, big, NULL), MOE_ERR_INVALID_ARG);
    moe_shape s136 = shape(64, 136, 4, 16, 4);
    EXPECT(dispatch(&s136, MOE_FP8_E4M3, A, 256, big, A), MOE_ERR_INVALID_ARG);

    EXPECT(combine(&s, A, -1, A), MOE_ERR_INVALID_ARG);
    EXPECT(combine(&s, NULL, 1, A), MOE_ERR_INVALID_ARG);
    EXPECT(combine(&s, A2, 1, A), MOE_ERR_INVALID_ARG);
    EXPECT(combine(&s, A, 1, (char*)A + 4), MOE_ERR_INVALID_ARG);
    moe_shape s0 = shape(0, 256, 4, 16, 4);
    EXPECT(combine(&s0, NULL, 0, NULL), MOE_OK); /* nothing to launch */

    EXPECT(moe_dispatch_ll(&s, MOE_BF16, A, A, A, big, 63, A, A, A, A, A, NULL), MOE_ERR_CAPACITY);
    EXPECT(moe_dispatch_ll(&s, MOE_BF16, A, A, A, big, -1, A, A, A, A, A, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch_ll(&s, MOE_BF16, A, A, A, 1, 64, A, A, A, A, A, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine_ll(&s, A, -1, A, A, A, A, NULL), MOE_ERR_INVALID_ARG);

    EXPECT(moe_combine_backward(&s, A, A, -1, A, A, A, A, A, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine_backward(&s, A, A, 1, A, A, A, A, NULL, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine_backward(&s0, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    EXPECT(moe_dispatch_backward(&s, A, -1, A, A, A, A, A, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch_backward(&s, A, 1, A, A, A, A, NULL, NULL), MOE_ERR_INVALID_ARG); /* grad_topk_w NULL alone */

    EXPECT(moe_encode_e4m3(A, A, -1, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_encode_e4m3(NULL, A, 4, NULL), MOE_ERR_INVALID_ARG);
    EXPECT(moe_encode_e4m3(NULL, NULL, 0, NULL), MOE_OK);

    moe_shape sr = shape(64, 256, 4, 64, 4);
    const moe_router bad_routers[] = {{7, 1, 1}, {MOE_GATE_SOFTMAX, 3, 1}, {MOE_GATE_SOFTMAX, 16, 2},
                                      {MOE_GATE_SOFTMAX, 2, 3}, {MOE_GATE_SOFTMAX, 2, 0}};
    for (size_t i = 0; i < sizeof(bad_routers) / sizeof(bad_routers[0]); ++i)
      if (moe_route_layout(&sr, &bad_routers[i], A, A, A, A, A, A, A, big, NULL) == MOE_OK) {
        fprintf(stderr, "router %zu accepted\n", i);
        ++failures;
      }
    EXPECT(moe_route_layout(&sr, NULL, A, A, A, A, A, A, A, big, NULL), MOE_ERR_INVALID_ARG);
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("host checks: all passed\n");
  return 0;
}
