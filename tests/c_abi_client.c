/*
 * A plain C client of libmoe_ep.so: no torch, no C++, only the header and the HIP runtime.
 *
 * It builds a small batch with known routing, runs layout -> dispatch (bf16) -> combine through
 * the C ABI on device memory it allocates itself, and checks results it can predict exactly:
 *   - token t names experts (t % E) and ((t + 1) % E), weights 1.0 and 0.0, k = 2, R = 4, E = 8;
 *   - combining the received rows back (y = recv_x) must return x bit for bit, because the
 *     weight-1 slot contributes x exactly and the weight-0 slot adds +0;
 *   - the per-rank token counts follow from the routing by hand.
 * Exit status 0 on success; prints what failed otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_ep.h"

#define CHECK_HIP(x)                                                  \
  do {                                                                \
    hipError_t e_ = (x);                                              \
    if (e_ != hipSuccess) {                                           \
      fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
      return 2;                                                       \
    }                                                                 \
  } while (0)

#define CHECK_MOE(x)                                                                   \
  do {                                                                                 \
    moe_status s_ = (x);                                                               \
    if (s_ != MOE_OK) {                                                                \
      fprintf(stderr, "%s failed: %s\n", #x, moe_status_string(s_));                 \
      return 3;                                                                        \
    }                                                                                  \
  } while (0)

int main(void) {
  enum { T = 200, H = 256, K = 2, E = 8, R = 4, L = E / R };
  moe_shape shape = {T, H, K, E, R};
  const int32_t cap = moe_max_recv_rows(&shape);
  const size_t ws_bytes = moe_workspace_bytes(&shape);
  if (cap != T * 2 || ws_bytes == 0) {
    fprintf(stderr, "bad sizes: cap %d workspace %zu\n", cap, ws_bytes);
    return 1;
  }

  /* host inputs */
  static uint16_t x[T * H];
  static int32_t idx[T * K];
  static float w[T * K];
  for (int t = 0; t < T; ++t) {
    for (int c = 0; c < H; ++c) x[t * H + c] = (uint16_t)(0x3f80u + ((t * 31 + c * 7) & 0x7f));  /* bf16 in [1, 2) */
    idx[t * K + 0] = t % E;
    idx[t * K + 1] = (t + 1) % E;
    w[t * K + 0] = 1.0f;
    w[t * K + 1] = 0.0f;
  }
  /* expected per-rank counts: token t reaches ranks (t % E) / L and ((t + 1) % E) / L */
  int32_t want_tpr[R] = {0};
  for (int t = 0; t < T; ++t) {
    const int r0 = (t % E) / L, r1 = ((t + 1) % E) / L;
    want_tpr[r0] += 1;
    if (r1 != r0) want_tpr[r1] += 1;
  }

  /* device buffers */
  uint16_t *dx, *drecv, *dout;
  int32_t *didx, *dtpr, *dtpe, *dsrc, *dridx, *doffs, *dsend, *dn;
  float *dw, *drw;
  uint8_t* dmask;
  void* dws;
  CHECK_HIP(hipMalloc((void**)&dx, sizeof(x)));
  CHECK_HIP(hipMalloc((void**)&didx, sizeof(idx)));
  CHECK_HIP(hipMalloc((void**)&dw, sizeof(w)));
  CHECK_HIP(hipMalloc((void**)&dtpr, R * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dtpe, E * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dmask, T * R));
  CHECK_HIP(hipMalloc(&dws, ws_bytes));
  CHECK_HIP(hipMalloc((void**)&drecv, (size_t)cap * H * sizeof(uint16_t)));
  CHECK_HIP(hipMalloc((void**)&dsrc, cap * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dridx, (size_t)cap * K * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&drw, (size_t)cap * K * sizeof(float)));
  CHECK_HIP(hipMalloc((void**)&doffs, (R + 1) * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dsend, T * R * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dn, sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dout, sizeof(x)));
  CHECK_HIP(hipMemcpy(dx, x, sizeof(x), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(didx, idx, sizeof(idx), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw, w, sizeof(w), hipMemcpyHostToDevice));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_MOE(moe_get_dispatch_layout(&shape, didx, dtpr, dtpe, dmask, dws, ws_bytes, stream));
  CHECK_MOE(moe_dispatch(&shape, MOE_BF16, dx, didx, dw, dws, ws_bytes, cap, drecv, NULL, dsrc, dridx, drw, doffs,
                         dsend, dn, stream));
  int32_t n = 0;
  CHECK_HIP(hipMemcpyAsync(&n, dn, sizeof(n), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_MOE(moe_combine(&shape, drecv, n, didx, dw, dsend, dout, stream));

  static uint16_t out[T * H];
  int32_t tpr[R];
  CHECK_HIP(hipMemcpyAsync(out, dout, sizeof(out), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipMemcpyAsync(tpr, dtpr, sizeof(tpr), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  int fails = 0;
  int32_t total = 0;
  for (int r = 0; r < R; ++r) {
    total += want_tpr[r];
    if (tpr[r] != want_tpr[r]) {
      fprintf(stderr, "tokens_per_rank[%d] = %d, want %d\n", r, tpr[r], want_tpr[r]);
      ++fails;
    }
  }
  if (n != total) {
    fprintf(stderr, "num_recv = %d, want %d\n", n, total);
    ++fails;
  }
  if (memcmp(out, x, sizeof(x)) != 0) {
    fprintf(stderr, "combine of the received rows did not return x\n");
    ++fails;
  }
  hipFree(dx); hipFree(didx); hipFree(dw); hipFree(dtpr); hipFree(dtpe); hipFree(dmask); hipFree(dws);
  hipFree(drecv); hipFree(dsrc); hipFree(dridx); hipFree(drw); hipFree(doffs); hipFree(dsend); hipFree(dn);
  hipFree(dout);
  hipStreamDestroy(stream);
  if (fails) return 1;
  printf("c abi client: layout, dispatch and combine through the C ABI match (num_recv %d)\n", n);
  return 0;
}
