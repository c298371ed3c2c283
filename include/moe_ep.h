/*
 * moe_ep.h — C ABI of the MI355X (gfx950) MoE expert-parallel dispatch/combine library.
 *
 * The library computes, on one GPU, the data-parallel core of expert-parallel
 * MoE communication as DeepEP describes it:
 *
 *   1. dispatch layout  — top-k expert ids -> per-rank and per-expert token
 *                         counts and the is_token_in_rank mask;
 *   2. dispatch         — each token's hidden row is packed, once per distinct
 *                         destination rank, into that rank's receive segment
 *                         (bf16 bit copy, or FP8 E4M3 with one fp32 scale per
 *                         128 channels);
 *   3. combine          — expert outputs are gathered back to their source
 *                         tokens as a top-k weighted fp32 sum, rounded to bf16.
 *
 * Passages followed (page titles as printed on the pages):
 *   [overlap notes]  "DeepEP：年度总结中的计算通信重叠摘记" (notes.kuangjux.top),
 *                    section 节点内通信 (intranode communication): only ranks
 *                    owning a selected expert receive a token (the
 *                    is_token_in_rank matrix), dispatch may carry FP8, and
 *                    dispatch and combine are the two measured exchange steps.
 *   [rocSHMEM notes] mlqm.cn notes on rocSHMEM and the RDMA buffer, section 3.2:
 *                    the exchange buffer holds packed outgoing rows and
 *                    received rows, is reused by combine, is allocated once
 *                    and sized for the worst case.
 *   [DeepEP overview] "DeepEP：面向MoE的高吞吐低延迟GPU通信库" (ssnai.com):
 *                    dispatch/combine kernels with FP8 and stream-ordered use.
 *
 * Logical ranks: the R destination ranks are R contiguous segments of one
 * receive buffer in this GPU's memory (rank r's rows are
 * [rank_offsets[r], rank_offsets[r+1])).  Expert e lives on rank e / L,
 * L = E / R.  Expert ids outside [0, E) are masked: every step skips them.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All array pointers are DEVICE pointers owned by the caller; the library
 *   allocates nothing and keeps no state between calls.  Outputs must not
 *   alias inputs.  An array pointer may be NULL exactly when the array has
 *   no elements (T == 0, capacity 0, no rows of y).  `shape` is a HOST
 *   pointer, read during the call only.
 * - Layout is row-major and densely packed.  bf16 values are passed as raw
 *   16-bit patterns.  Payload pointers (x, recv_x, y, out) must be 16-byte
 *   aligned; int32/float arrays 4-byte aligned.
 * - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *   without waiting; nothing is read back to the host.
 * - Arguments are checked on the host before anything is enqueued; on any
 *   error nothing is launched and no memory is touched.  A launch failure
 *   reported by the runtime returns MOE_ERR_HIP.
 * - Limits: 0 <= T <= 2^30, 1 <= k <= 32, 1 <= R <= 64, R <= E <= 4096, E % R == 0,
 *   H > 0 and H % 8 == 0 (H % 128 == 0 for FP8), T*k and T*R below 2^31.
 */
#ifndef MOE_EP_H_
#define MOE_EP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_shape {
  int32_t num_tokens;  /* T: tokens of this source batch */
  int32_t hidden;      /* H: channels per token row */
  int32_t num_topk;    /* k: expert slots per token */
  int32_t num_experts; /* E */
  int32_t num_ranks;   /* R: logical destination ranks */
} moe_shape;

typedef enum moe_dtype {
  MOE_BF16 = 0,     /* receive rows are bf16 bit copies of x */
  MOE_FP8_E4M3 = 1, /* receive rows are OCP E4M3 bytes + fp32 scale per 128 channels */
  MOE_DTYPE_MAX_ENUM = 0x7fffffff /* not a dtype: makes the type 32 bits wide and every
                                     non-negative value a caller passes representable (rejected
                                     with MOE_ERR_INVALID_ARG unless listed above) */
} moe_dtype;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, workspace too small */
  MOE_ERR_CAPACITY = 2,    /* receive capacity below T * min(k, R) */
  MOE_ERR_UNSUPPORTED = 3, /* shape outside the limits above */
  MOE_ERR_HIP = 4,         /* the HIP runtime reported a launch error */
  MOE_STATUS_MAX_ENUM = 0x7fffffff /* not a status: makes the type 32 bits wide */
} moe_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status status);

/* Bytes of device workspace the layout writes and dispatch reads for `shape`
 * (0 if the shape is invalid).  The workspace is the dispatch plan: the
 * per-token rank bitmasks, per-64-token-chunk prefix counts per rank and the
 * rank offsets.  Its first bytes also hold words through which the blocks of
 * one launch hand the plan's last step to the block that finishes last:
 * ZERO-FILL A NEW WORKSPACE ONCE before its first use (hipMemset); every call
 * leaves those words zero again, so a workspace is reused without clearing.
 * Calls sharing a workspace must not run concurrently (they already share the
 * plan).  The plan carries no state across different layouts. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Worst-case receive rows, T * min(k, R): every token sent to min(k, R)
 * distinct ranks.  [rocSHMEM notes 3.2: the buffer is sized once for the worst
 * case.]  Returns -1 if the shape is invalid. */
int32_t moe_max_recv_rows(const moe_shape* shape);

/* Dispatch layout.  [overlap notes, 节点内通信: the is_token_in_rank filter.]
 *
 *   topk_idx          in  int32[T, k]   expert id per slot (ids outside [0,E) masked)
 *   tokens_per_rank   out int32[R]      number of tokens sent to each rank
 *   tokens_per_expert out int32[E]      number of valid slots naming each expert
 *   is_token_in_rank  out uint8[T, R]   1 iff a valid slot of token t names an expert of rank r, else 0
 *   workspace         out bytes[ws]     dispatch plan consumed by moe_dispatch
 *                                       (workspace_bytes >= moe_workspace_bytes(shape);
 *                                       zero-filled once when allocated, see above)
 *
 * One launch at every size: up to 1024 tokens one block does everything; above,
 * blocks of 256 tokens count in parallel and the block that finishes last takes
 * the prefix sums (no block waits for another).
 */
moe_status moe_get_dispatch_layout(const moe_shape* shape, const int32_t* topk_idx,
                                   int32_t* tokens_per_rank, int32_t* tokens_per_expert,
                                   uint8_t* is_token_in_rank, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Gate of a router fused with the layout (moe_route_layout). */
typedef enum moe_gate {
  MOE_GATE_SOFTMAX = 0, /* w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k selected */
  MOE_GATE_SIGMOID = 1  /* w_j = s(l_j) / sum_i s(l_i), s(x) = 1 / (1 + exp(-x)), over the k selected */
} moe_gate;

typedef struct moe_router {
  int32_t gate;        /* moe_gate */
  int32_t num_groups;  /* G: experts form G equal contiguous groups; 1 = no group limit */
  int32_t topk_groups; /* groups kept per token, 1 <= topk_groups <= G */
} moe_router;

/* Top-k gating fused with the dispatch layout.  [overlap notes, 节点内通信: top-k
 * runs together with the sparse exchange, no CPU step between them; section
 * 计算-通信重叠: DeepSeek's group-limited gating.]
 *
 * Per token: with G > 1, each group is scored by its largest logit and the
 * topk_groups best groups are kept (equal scores: the lower group first); the k
 * largest logits among the kept groups' experts are selected, equal logits in
 * ascending id order (-0.0 equals +0.0), and written in descending order of
 * logit; the weights follow `gate` in fp32.  Then everything
 * moe_get_dispatch_layout computes is computed from those ids, so moe_dispatch
 * can follow directly.
 *
 *   router            in  gate, num_groups, topk_groups
 *   logits            in  float[T, E]     finite router logits (NaN: selection unspecified)
 *   topk_idx          out int32[T, k]     selected expert ids, slot order
 *   topk_w            out float[T, k]     gate weights
 *   tokens_per_rank, tokens_per_expert, is_token_in_rank, workspace: as moe_get_dispatch_layout
 *
 * Limits: E % 8 == 0, k <= 16, num_groups in {1, 2, 4, 8}
 * (MOE_ERR_UNSUPPORTED otherwise); E % num_groups == 0 and
 * k <= topk_groups * E / num_groups (MOE_ERR_INVALID_ARG otherwise).
 */
moe_status moe_route_layout(const moe_shape* shape, const moe_router* router, const float* logits,
                            int32_t* topk_idx, float* topk_w, int32_t* tokens_per_rank,
                            int32_t* tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Routing, layout and dispatch in one call.  [overlap notes, 节点内通信: DeepEP
 * runs top-k together with the sparse exchange so that no CPU step separates
 * them.]
 *
 * Writes everything moe_route_layout and then moe_dispatch (on the ids and
 * weights just computed) write for the same arguments -- topk_idx, topk_w,
 * tokens_per_rank, tokens_per_expert, is_token_in_rank, the plan in
 * `workspace`, the receive rows and their metadata, rank_offsets, send_row and
 * num_recv -- with identical values.  Arguments, limits and errors are the
 * union of the two calls' (topk_idx and topk_w are outputs here).  For
 * 1 <= T <= 1024 one kernel does all of it: its first blocks route, the last of
 * them to finish completes the plan, and the remaining blocks, which load
 * their rows of x meanwhile, pack the rows once the plan is complete (no
 * block waits for a block that could be waiting itself); otherwise the two
 * calls' launches run back to back.
 */
moe_status moe_route_dispatch(const moe_shape* shape, const moe_router* router, moe_dtype dtype, const float* logits,
                              const void* x, int32_t* topk_idx, float* topk_w, int32_t* tokens_per_rank,
                              int32_t* tokens_per_expert, uint8_t* is_token_in_rank, void* workspace,
                              size_t workspace_bytes, int32_t recv_capacity, void* recv_x, float* recv_scales,
                              int32_t* recv_src_idx, int32_t* recv_topk_idx, float* recv_topk_w,
                              int32_t* rank_offsets, int32_t* send_row, int32_t* num_recv, hipStream_t stream);

/* Dispatch.  [overlap notes, 节点内通信: filtered send, FP8 transport;
 * rocSHMEM notes 3.2: rows packed into a preallocated receive buffer.]
 *
 * Receive row of (token t, rank r) = rank_offsets[r] + number of tokens t' < t
 * that also go to r: segments in rank order, rows in ascending token order.
 *
 *   dtype          MOE_BF16 or MOE_FP8_E4M3
 *   x              in  bf16[T, H]
 *   topk_idx       in  int32[T, k]     the ids the layout was computed from
 *   topk_w         in  float[T, k]     gate weights
 *   workspace      in  bytes[ws]       written by moe_get_dispatch_layout for the same topk_idx
 *   recv_capacity      rows allocated in the receive arrays; >= T * min(k, R)
 *   recv_x         out bf16[cap, H] (MOE_BF16) or uint8[cap, H] (MOE_FP8_E4M3)
 *   recv_scales    out float[cap, H/128]  dequantisation scale s per 128-channel
 *                      block (x ~= decode(q) * s), s = fl32(max(amax, 1e-4) / 448),
 *                      q = E4M3_RNE(fl32(x / s)); NULL allowed (and ignored) for MOE_BF16
 *   recv_src_idx   out int32[cap]      source token of each receive row
 *   recv_topk_idx  out int32[cap, k]   local expert id (e - r*L) of slot j if it
 *                                      names an expert of the row's rank, else -1
 *   recv_topk_w    out float[cap, k]   weight of slot j where recv_topk_idx >= 0, else +0.0
 *   rank_offsets   out int32[R + 1]    segment starts; rank_offsets[R] = number of rows
 *   send_row       out int32[T, R]     receive row of (t, r), or -1 if t is not sent to r
 *   num_recv       out int32[1]        number of receive rows written (= rank_offsets[R])
 *
 * Rows at or beyond num_recv are not written.
 */
moe_status moe_dispatch(const moe_shape* shape, moe_dtype dtype, const void* x,
                        const int32_t* topk_idx, const float* topk_w, const void* workspace,
                        size_t workspace_bytes, int32_t recv_capacity, void* recv_x,
                        float* recv_scales, int32_t* recv_src_idx, int32_t* recv_topk_idx,
                        float* recv_topk_w, int32_t* rank_offsets, int32_t* send_row,
                        int32_t* num_recv, hipStream_t stream);

/* Layout and dispatch in one call.  [overlap notes, 节点内通信: filtered send;
 * rocSHMEM notes 3.2: rows packed into a preallocated receive buffer.]
 *
 * Writes everything moe_get_dispatch_layout and then moe_dispatch write for the
 * same arguments -- tokens_per_rank, tokens_per_expert, is_token_in_rank, the
 * plan in `workspace` (so that a later moe_dispatch with this workspace is
 * valid), the receive rows, their metadata, rank_offsets, send_row and
 * num_recv -- with identical values.  Arguments, limits and errors are the
 * union of the two calls'.  For T <= 1024 and hidden <= 16384 one kernel does
 * both steps (every block recounts the batch's rank bitmasks, so no launch
 * boundary separates the prefix sums from the packing); otherwise the two
 * calls' launches run back to back.
 */
moe_status moe_layout_dispatch(const moe_shape* shape, moe_dtype dtype, const void* x, const int32_t* topk_idx,
                               const float* topk_w, int32_t* tokens_per_rank, int32_t* tokens_per_expert,
                               uint8_t* is_token_in_rank, void* workspace, size_t workspace_bytes,
                               int32_t recv_capacity, void* recv_x, float* recv_scales, int32_t* recv_src_idx,
                               int32_t* recv_topk_idx, float* recv_topk_w, int32_t* rank_offsets,
                               int32_t* send_row, int32_t* num_recv, hipStream_t stream);

/* moe_layout_dispatch without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The dispatch plan lives in a static
 * device array of the library, 4 MiB per device (held until the process
 * ends); shapes whose plan (moe_workspace_bytes) exceeds 4 MiB are rejected
 * with MOE_ERR_UNSUPPORTED -- about 300,000 tokens at 256 experts and 64
 * ranks.  The call allocates nothing and otherwise behaves exactly as
 * moe_layout_dispatch: same arguments (minus the workspace), outputs, limits
 * and errors; MOE_ERR_HIP if the array's device address cannot be obtained.
 * All calls on one device share the array: calls that overlap in time on one
 * device (on different streams, or from several threads) race and give
 * undefined results.  Each call leaves the array ready for the next. */
moe_status moe_layout_dispatch_noalloc(const moe_shape* shape, moe_dtype dtype, const void* x,
                                       const int32_t* topk_idx, const float* topk_w, int32_t* tokens_per_rank,
                                       int32_t* tokens_per_expert, uint8_t* is_token_in_rank, int32_t recv_capacity,
                                       void* recv_x, float* recv_scales, int32_t* recv_src_idx,
                                       int32_t* recv_topk_idx, float* recv_topk_w, int32_t* rank_offsets,
                                       int32_t* send_row, int32_t* num_recv, hipStream_t stream);

/* The E4M3 rounding the FP8 dispatch applies to x / s, on its own.
 * [overlap notes, 节点内通信: FP8 transport.]
 *
 * codes[i] = the nearest OCP E4M3 ("fn": bias 7, max 448) value to values[i],
 * ties to the even code, sign kept (negative values that round to zero give
 * 0x80).  Defined for finite |values[i]| < 464, the range the dispatch's
 * per-128-channel scaling produces; other inputs give unspecified codes.
 *
 *   values  in  float[n]   device memory
 *   codes   out uint8[n]   device memory
 *   n           number of values; 0 launches nothing
 *
 * MOE_ERR_INVALID_ARG for n < 0 or a NULL array with n > 0.
 */
moe_status moe_encode_e4m3(const float* values, uint8_t* codes, int64_t n, hipStream_t stream);

/* Combine.  [overlap notes, 节点内通信: combine; rocSHMEM notes 3.2: the
 * receive buffer is reused for the returning expert outputs.]
 *
 * out[t, c] = BF16_RNE(acc) with acc = +0 and, for j = 0..k-1 in order over
 * valid slots, acc = fl32(acc + fl32(topk_w[t, j] * y[send_row[t, e_tj / L], c]))
 * (no fused multiply-add).  Tokens without a valid slot get +0.
 *
 *   y          in  bf16[num_y_rows, H]  expert outputs in receive-row order
 *   num_y_rows     rows of y; slots whose row is outside [0, num_y_rows) are skipped
 *   topk_idx   in  int32[T, k]
 *   topk_w     in  float[T, k]
 *   send_row   in  int32[T, R]          from moe_dispatch
 *   out        out bf16[T, H]
 */
moe_status moe_combine(const moe_shape* shape, const void* y, int32_t num_y_rows,
                       const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                       void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Low-latency (per-expert) layout.  [DeepEP overview: the low-latency kernels
 * for decoding; overlap notes, 节点间通信: the low-latency mode.]  The receive
 * side keeps one fixed-capacity buffer per expert: buffers are [E, cap, ...],
 * i.e. R ranks x [L, cap, ...] as each rank would hold its local experts.
 * One receive row per (token, distinct valid expert); token t's row in expert
 * e's buffer is pos(t, e) = number of tokens t' < t naming e.  The layout is
 * computed inside moe_dispatch_ll (no separate layout call).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_dispatch_ll needs for `shape` (0 if invalid). */
size_t moe_ll_workspace_bytes(const moe_shape* shape);

/* Low-latency dispatch.
 *
 *   dtype            MOE_BF16 or MOE_FP8_E4M3 (same per-128 scaling as moe_dispatch)
 *   x                in  bf16[T, H]
 *   topk_idx         in  int32[T, k]
 *   workspace        scratch, >= moe_ll_workspace_bytes(shape) bytes, 256-byte aligned
 *   expert_capacity      rows per expert buffer; >= T (else MOE_ERR_CAPACITY)
 *   recv_x           out bf16 or uint8 [E, cap, H]
 *   recv_scales      out float[E, cap, H/128] (FP8 only; NULL allowed for MOE_BF16)
 *   recv_src_idx     out int32[E, cap]   source token of each written row
 *   recv_count       out int32[E]        rows written per expert (distinct tokens naming it)
 *   slot_pos         out int32[T, k]     pos(t, e_tj) for valid slots (shared by repeated
 *                                        ids of one token), else -1: the combine handle
 *
 * Rows at or beyond recv_count[e] are not written.
 */
moe_status moe_dispatch_ll(const moe_shape* shape, moe_dtype dtype, const void* x, const int32_t* topk_idx,
                           void* workspace, size_t workspace_bytes, int32_t expert_capacity, void* recv_x,
                           float* recv_scales, int32_t* recv_src_idx, int32_t* recv_count,
                           int32_t* slot_pos, hipStream_t stream);

/* Low-latency combine: out[t] = BF16_RNE(sum over valid slots j, ascending, in fp32 without
 * fused multiply-add, of topk_w[t, j] * y[e_tj, slot_pos[t, j]]).
 *
 *   y                in  bf16[E, cap, H]  expert outputs in the per-expert layout
 *   expert_capacity      cap of y
 *   topk_idx, topk_w in  int32/float[T, k]
 *   slot_pos         in  int32[T, k]      from moe_dispatch_ll
 *   out              out bf16[T, H]
 */
moe_status moe_combine_ll(const moe_shape* shape, const void* y, int32_t expert_capacity,
                          const int32_t* topk_idx, const float* topk_w, const int32_t* slot_pos,
                          void* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward (training).  [DeepEP overview: the library serves training; its
 * backward path needs its own integration.]  Each is the adjoint of the
 * forward step above, on the rank layout.
 * ------------------------------------------------------------------------ */

/* Combine backward.
 *   grad_out     in  bf16[T, H]             gradient of the combine output
 *   y            in  bf16[num_y_rows, H]    the combine's expert outputs
 *   topk_idx, topk_w, send_row              as given to moe_combine
 *   grad_y       out bf16[num_y_rows, H]    row send_row[t, r] = BF16_RNE(fp32 sum over the
 *                                           slots j of t on rank r, ascending, of
 *                                           fl32(topk_w[t, j] * grad_out[t])); rows no slot
 *                                           refers to are not written
 *   grad_topk_w  out float[T, k]            <grad_out[t], y[row(t, j)]> summed in fp32 in a
 *                                           fixed order (deterministic); 0 for invalid slots
 *                                           and for slots whose row is not below num_y_rows
 * With num_y_rows == 0, y and grad_y may be NULL: nothing is written to grad_y and every
 * grad_topk_w is +0.
 */
moe_status moe_combine_backward(const moe_shape* shape, const void* grad_out, const void* y, int32_t num_y_rows,
                                const int32_t* topk_idx, const float* topk_w, const int32_t* send_row,
                                void* grad_y, float* grad_topk_w, hipStream_t stream);

/* Dispatch backward.
 *   grad_recv_x       in  bf16[num_recv_rows, H]   gradient w.r.t. the received rows (FP8
 *                                                  dispatch is passed straight through)
 *   grad_recv_topk_w  in  float[num_recv_rows, k]  gradient w.r.t. recv_topk_w, or NULL
 *   topk_idx, send_row                             as given to / returned by moe_dispatch (a
 *                                                  token has at most min(k, R) valid send_row
 *                                                  entries; further ones are not read)
 *   grad_x            out bf16[T, H]    BF16_RNE(fp32 sum over ranks r ascending of
 *                                       grad_recv_x[send_row[t, r]]); +0 for unsent tokens
 *   grad_topk_w       out float[T, k]   grad_recv_topk_w[row(t, j), j], 0 for invalid slots;
 *                                       NULL exactly when grad_recv_topk_w is NULL
 */
moe_status moe_dispatch_backward(const moe_shape* shape, const void* grad_recv_x, int32_t num_recv_rows,
                                 const float* grad_recv_topk_w, const int32_t* topk_idx,
                                 const int32_t* send_row, void* grad_x, float* grad_topk_w,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * Compute-unit budget.  [overlap notes, 节点内通信: DeepEP gives its exchange
 * kernels a fixed share of the SMs (20 of 132) so that expert computation
 * overlaps on the rest; DeepEP overview: Buffer.set_num_sms trades exchange
 * latency against compute.]  The MI355X equivalent is a stream whose kernels
 * may only run on a chosen set of CUs.  Launches of this library on a stream
 * made by moe_stream_create_cu_range size their persistent grids to that
 * stream's CUs (looked up in a table the library keeps, not queried from the
 * runtime per call); any other stream counts as unrestricted (results are
 * the same either way; only the grid size differs).
 *
 * CU-mask bit i of a stream belongs to XCD (i mod number of XCDs) on MI355X,
 * and every XCD must keep at least one CU; so the range [first_cu,
 * first_cu + num_cus) must consist of multiples of the XCD count (8), which
 * gives every XCD the same number of CUs.
 * ------------------------------------------------------------------------ */

/* Creates (non-blocking, default priority) a stream restricted to CUs
 * [first_cu, first_cu + num_cus) of the current device.  first_cu == 0 with
 * num_cus <= 0 or >= the CU count gives an unrestricted stream.  The caller
 * destroys it with moe_stream_destroy.  MOE_ERR_INVALID_ARG for a range that
 * is not a multiple of the XCD count or exceeds the device;
 * MOE_ERR_UNSUPPORTED with 64 restricted streams already alive. */
moe_status moe_stream_create_cu_range(int32_t first_cu, int32_t num_cus, hipStream_t* stream);

/* Destroys a stream made by moe_stream_create_cu_range. */
moe_status moe_stream_destroy(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EP_H_ */
