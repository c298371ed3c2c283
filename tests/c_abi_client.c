/*
 * A plain C client of libmoe_ep.so: no torch, no C++, only the header and the HIP runtime.
 *
 * It builds a small batch with known routing, runs layout -> dispatch (bf16) -> combine, the
 * dispatch backward, the low-latency dispatch and combine, and the E4M3 encoder through the C ABI on
 * device memory it allocates itself, and checks results it can predict exactly:
 *   - token t names experts (t % E) and ((t + 1) % E), weights 1.0 and 0.0, k = 2, R = 4, E = 8;
 *   - combining the received rows back (y = recv_x) must return x bit for bit, because the
 *     weight-1 slot contributes x exactly and the weight-0 slot adds +0 (both layouts);
 *   - the per-rank and per-expert counts follow from the routing by hand;
 *   - the dispatch backward of the received rows is x times the number of distinct ranks;
 *   - E4M3 codes of exactly representable values, ties and signed zero are known;
 *   - layout and dispatch as one call (moe_layout_dispatch) give the two calls' rows and handle.
 * It also times the host side of each entry point: 1000 calls enqueued back to back with no
 * synchronisation inside the loop, printed as "host_us_per_call <name> <microseconds>" (argument
 * checks plus kernel enqueue; the GPU work itself is not waited for).
 * Exit status 0 on success; prints what failed otherwise.
 */
#define _POSIX_C_SOURCE 199309L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

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
  CHECK_HIP(hipMemset(dws, 0, ws_bytes)); /* a new workspace is zero-filled once */
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

  /* dispatch backward of the received rows: each token gets x once per distinct rank it went to,
   * i.e. x or 2x (exact: x is in [1, 2), so 2x adds one to the bf16 exponent field) */
  uint16_t* dgx;
  CHECK_HIP(hipMalloc((void**)&dgx, sizeof(x)));
  CHECK_MOE(moe_dispatch_backward(&shape, drecv, n, NULL, didx, dsend, dgx, NULL, stream));
  static uint16_t gx[T * H];
  CHECK_HIP(hipMemcpyAsync(gx, dgx, sizeof(gx), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  for (int t = 0; t < T && fails < 8; ++t) {
    const int two = (t % E) / L != ((t + 1) % E) / L;
    for (int c = 0; c < H; ++c) {
      const uint16_t want = (uint16_t)(x[t * H + c] + (two ? 0x80 : 0));
      if (gx[t * H + c] != want) {
        fprintf(stderr, "dispatch backward: token %d channel %d = 0x%04x, want 0x%04x\n", t, c, gx[t * H + c], want);
        ++fails;
        break;
      }
    }
  }

  /* low-latency layout: per-expert buffers [E, T, H]; combining them back with weights 1 and 0
   * returns x bit for bit */
  const size_t ll_ws = moe_ll_workspace_bytes(&shape);
  void* dllws;
  uint16_t *dllx, *dllout;
  int32_t *dllsrc, *dllcnt, *dllpos;
  CHECK_HIP(hipMalloc(&dllws, ll_ws));
  CHECK_HIP(hipMalloc((void**)&dllx, (size_t)E * T * H * sizeof(uint16_t)));
  CHECK_HIP(hipMalloc((void**)&dllsrc, (size_t)E * T * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dllcnt, E * sizeof(int32_t)));
  CHECK_HIP(hipMalloc((void**)&dllpos, sizeof(idx)));
  CHECK_HIP(hipMalloc((void**)&dllout, sizeof(x)));
  CHECK_MOE(moe_dispatch_ll(&shape, MOE_BF16, dx, didx, dllws, ll_ws, T, dllx, NULL, dllsrc, dllcnt, dllpos, stream));
  CHECK_MOE(moe_combine_ll(&shape, dllx, T, didx, dw, dllpos, dllout, stream));
  int32_t cnt[E];
  CHECK_HIP(hipMemcpyAsync(out, dllout, sizeof(out), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipMemcpyAsync(cnt, dllcnt, sizeof(cnt), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  for (int e = 0; e < E; ++e) {
    int want = 0; /* tokens naming e: t % E == e or (t + 1) % E == e */
    for (int t = 0; t < T; ++t) want += (t % E == e) || ((t + 1) % E == e);
    if (cnt[e] != want) {
      fprintf(stderr, "recv_count[%d] = %d, want %d\n", e, cnt[e], want);
      ++fails;
    }
  }
  if (memcmp(out, x, sizeof(x)) != 0) {
    fprintf(stderr, "low-latency combine of the received rows did not return x\n");
    ++fails;
  }

  /* layout and dispatch as one call: the same counts, rows and handle as the two calls above */
  {
    int32_t *tpr2, *tpe2, *src2, *ridx2, *offs2, *send2, *n2;
    uint8_t* mask2;
    uint16_t* recv2;
    float* rw2;
    void* ws2;
    CHECK_HIP(hipMalloc((void**)&tpr2, R * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&tpe2, E * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&mask2, T * R));
    CHECK_HIP(hipMalloc(&ws2, ws_bytes));
    CHECK_HIP(hipMalloc((void**)&recv2, (size_t)cap * H * sizeof(uint16_t)));
    CHECK_HIP(hipMalloc((void**)&src2, cap * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&ridx2, (size_t)cap * K * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&rw2, (size_t)cap * K * sizeof(float)));
    CHECK_HIP(hipMalloc((void**)&offs2, (R + 1) * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&send2, T * R * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&n2, sizeof(int32_t)));
    CHECK_MOE(moe_layout_dispatch(&shape, MOE_BF16, dx, didx, dw, tpr2, tpe2, mask2, ws2, ws_bytes, cap, recv2, NULL,
                                  src2, ridx2, rw2, offs2, send2, n2, stream));
    static int32_t sa[T * R], sb[T * R];
    static uint16_t ra[T * 2 * H], rb[T * 2 * H];
    int32_t nb = -1;
    CHECK_HIP(hipMemcpyAsync(sa, dsend, sizeof(sa), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(sb, send2, sizeof(sb), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(ra, drecv, (size_t)n * H * sizeof(uint16_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(rb, recv2, (size_t)n * H * sizeof(uint16_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(&nb, n2, sizeof(nb), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (nb != n || memcmp(sa, sb, sizeof(sa)) != 0 || memcmp(ra, rb, (size_t)n * H * sizeof(uint16_t)) != 0) {
      fprintf(stderr, "moe_layout_dispatch differs from the two calls (num_recv %d vs %d)\n", nb, n);
      ++fails;
    }
    hipFree(tpr2); hipFree(tpe2); hipFree(mask2); hipFree(ws2); hipFree(recv2); hipFree(src2); hipFree(ridx2);
    hipFree(rw2); hipFree(offs2); hipFree(send2); hipFree(n2);
  }

  /* the E4M3 rounding on its own: exact values, ties to even, signed zero, the largest code */
  const float fv[10] = {0.0f, -0.0f, 1.0f, -2.0f, 448.0f, 0x1p-9f, 0x1p-10f, 0x3p-10f, 1.0625f, 1.1875f};
  const uint8_t fwant[10] = {0x00, 0x80, 0x38, 0xC0, 0x7E, 0x01, 0x00, 0x02, 0x38, 0x3A};
  float* dfv;
  uint8_t* dfq;
  uint8_t fq[10];
  CHECK_HIP(hipMalloc((void**)&dfv, sizeof(fv)));
  CHECK_HIP(hipMalloc((void**)&dfq, sizeof(fq)));
  CHECK_HIP(hipMemcpy(dfv, fv, sizeof(fv), hipMemcpyHostToDevice));
  CHECK_MOE(moe_encode_e4m3(dfv, dfq, 10, stream));
  CHECK_HIP(hipMemcpyAsync(fq, dfq, sizeof(fq), hipMemcpyDeviceToHost, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  for (int i = 0; i < 10; ++i) {
    if (fq[i] != fwant[i]) {
      fprintf(stderr, "moe_encode_e4m3(%a) = 0x%02x, want 0x%02x\n", (double)fv[i], fq[i], fwant[i]);
      ++fails;
    }
  }
  /* host cost per call: reps enqueues of one entry point, no synchronisation in the loop */
  {
    enum { REPS = 1000 };
    static float logits[T * E];
    for (int i = 0; i < T * E; ++i) logits[i] = (float)((i * 37) % 101) / 101.0f;
    float *dlog, *dw2;
    int32_t *didx2, *dtpr3, *dtpe3;
    uint8_t* dmask3;
    void* dws3;
    CHECK_HIP(hipMalloc((void**)&dlog, sizeof(logits)));
    CHECK_HIP(hipMalloc((void**)&dw2, sizeof(w)));
    CHECK_HIP(hipMalloc((void**)&didx2, sizeof(idx)));
    CHECK_HIP(hipMalloc((void**)&dtpr3, R * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&dtpe3, E * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&dmask3, T * R));
    CHECK_HIP(hipMalloc(&dws3, ws_bytes));
    CHECK_HIP(hipMemset(dws3, 0, ws_bytes));
    CHECK_HIP(hipMemcpy(dlog, logits, sizeof(logits), hipMemcpyHostToDevice));
    CHECK_HIP(hipStreamSynchronize(stream));
    const moe_router router = {MOE_GATE_SOFTMAX, 1, 1};
    struct timespec t0, t1;
#define TIME_CALLS(name, call)                                                                          \
  do {                                                                                                 \
    clock_gettime(CLOCK_MONOTONIC, &t0);                                                               \
    for (int i_ = 0; i_ < REPS; ++i_) CHECK_MOE(call);                                                 \
    clock_gettime(CLOCK_MONOTONIC, &t1);                                                               \
    CHECK_HIP(hipStreamSynchronize(stream));                                                           \
    printf("host_us_per_call %s %.3f\n", name,                                                         \
           ((double)(t1.tv_sec - t0.tv_sec) * 1e6 + (double)(t1.tv_nsec - t0.tv_nsec) / 1e3) / REPS);   \
  } while (0)
    clock_gettime(CLOCK_MONOTONIC, &t0);
    for (int i = 0; i < REPS; ++i) CHECK_HIP(hipMemsetAsync(dfq, 0, 4, stream));
    clock_gettime(CLOCK_MONOTONIC, &t1);
    CHECK_HIP(hipStreamSynchronize(stream));
    printf("host_us_per_call hipMemsetAsync_4_bytes %.3f\n",
           ((double)(t1.tv_sec - t0.tv_sec) * 1e6 + (double)(t1.tv_nsec - t0.tv_nsec) / 1e3) / REPS);
    TIME_CALLS("moe_get_dispatch_layout", moe_get_dispatch_layout(&shape, didx, dtpr, dtpe, dmask, dws, ws_bytes,
                                                                  stream));
    TIME_CALLS("moe_dispatch", moe_dispatch(&shape, MOE_BF16, dx, didx, dw, dws, ws_bytes, cap, drecv, NULL, dsrc,
                                            dridx, drw, doffs, dsend, dn, stream));
    TIME_CALLS("moe_layout_dispatch", moe_layout_dispatch(&shape, MOE_BF16, dx, didx, dw, dtpr, dtpe, dmask, dws,
                                                          ws_bytes, cap, drecv, NULL, dsrc, dridx, drw, doffs,
                                                          dsend, dn, stream));
    TIME_CALLS("moe_combine", moe_combine(&shape, drecv, n, didx, dw, dsend, dout, stream));
    TIME_CALLS("moe_dispatch_backward", moe_dispatch_backward(&shape, drecv, n, NULL, didx, dsend, dgx, NULL,
                                                              stream));
    TIME_CALLS("moe_dispatch_ll", moe_dispatch_ll(&shape, MOE_BF16, dx, didx, dllws, ll_ws, T, dllx, NULL, dllsrc,
                                                  dllcnt, dllpos, stream));
    TIME_CALLS("moe_combine_ll", moe_combine_ll(&shape, dllx, T, didx, dw, dllpos, dllout, stream));
    TIME_CALLS("moe_encode_e4m3", moe_encode_e4m3(dfv, dfq, 10, stream));
    TIME_CALLS("moe_route_layout", moe_route_layout(&shape, &router, dlog, didx2, dw2, dtpr3, dtpe3, dmask3, dws3,
                                                    ws_bytes, stream));
    TIME_CALLS("moe_route_dispatch", moe_route_dispatch(&shape, &router, MOE_BF16, dlog, dx, didx2, dw2, dtpr3,
                                                        dtpe3, dmask3, dws3, ws_bytes, cap, drecv, NULL, dsrc,
                                                        dridx, drw, doffs, dsend, dn, stream));
#undef TIME_CALLS
    hipFree(dlog); hipFree(dw2); hipFree(didx2); hipFree(dtpr3); hipFree(dtpe3); hipFree(dmask3); hipFree(dws3);
  }

  hipFree(dgx); hipFree(dllws); hipFree(dllx); hipFree(dllsrc); hipFree(dllcnt); hipFree(dllpos); hipFree(dllout);
  hipFree(dfv); hipFree(dfq);
  hipFree(dx); hipFree(didx); hipFree(dw); hipFree(dtpr); hipFree(dtpe); hipFree(dmask); hipFree(dws);
  hipFree(drecv); hipFree(dsrc); hipFree(dridx); hipFree(drw); hipFree(doffs); hipFree(dsend); hipFree(dn);
  hipFree(dout);
  hipStreamDestroy(stream);
  if (fails) return 1;
  printf("c abi client: layout, dispatch, one-call layout+dispatch, combine, dispatch backward, low-latency "
         "dispatch/combine and E4M3 encoding through the C ABI match (num_recv %d)\n", n);
  return 0;
}
