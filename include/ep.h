/*
 * ep.h -- C ABI of the MI355X (gfx950) MoE expert-parallel dispatch/combine
 * library.
 *
 * The method is the one described in "Enabling trillion-parameter models on
 * AWS EFA" (Perplexity, 2025-11-04):
 *   - section "Dispatch and combine": dispatch receives the tokens and each
 *     token's experts from the model and moves every token to the ranks that
 *     host its experts; after the grouped GEMM, combine brings the results
 *     back to the source rank and forms the routing-weighted average;
 *     both halves are split into a sender and a receiver;
 *   - section "Send and receive buffers": per-expert token counts are
 *     exchanged first so that each sender can place its rows contiguously
 *     per peer (one bulk write per peer) and each receiver knows the offset
 *     at which every source lands; a receiver needs room for at most
 *     N * T * max(R, E/N) rows;
 *   - timing figures of section "Dispatch and combine": per-expert counts,
 *     then a running prefix sum gives the send-buffer offsets; the receiver
 *     shuffles its receive buffer into the grouped-GEMM input; the combine
 *     receiver accumulates the weighted tokens into the output tensor;
 *   - section "Evaluation": hidden 7168, block-scaled fp8 dispatch, bf16
 *     combine.
 *
 * One GPU holds all N ranks of the expert-parallel group ("virtual ranks"):
 * every rank's buffers live in that GPU's HBM and the network write is a
 * device-local copy. Every call handles all N ranks in one launch sequence.
 *
 * Notation: N ranks, T tokens per rank, H hidden size, E experts, R experts
 * per token, L = E / N experts per rank. Expert e lives on rank e / L as
 * local expert e % L. A slot is (s, t, k): source rank s, token t, choice k.
 *
 * Conventions shared by every call:
 *   - All buffers are device memory owned by the caller, contiguous and
 *     row-major in the shapes given below. The library allocates nothing and
 *     keeps no state between calls; it is re-entrant.
 *   - Row buffers (payload planes, expert outputs, combined tokens, partial
 *     sums, KV pools) and the plan workspace must start on a 16-byte
 *     boundary (EP_ERR_INVALID_ARG otherwise); rows are moved with 16-byte
 *     vector accesses and the plan's row-pair table is read 8 bytes at a
 *     time.
 *   - A buffer that ends before the extent a call needs (per its shapes)
 *     gives EP_ERR_INVALID_ARG when the runtime reports the allocation's
 *     range (hipMemGetAddressRange); a sub-range of a larger allocation can
 *     only be checked against that allocation's end.
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     The device is taken from the stream (not from the calling thread);
 *     buffers on another device give EP_ERR_DEVICE_MISMATCH.
 *   - Host-side checks fail fast with a negative return and enqueue nothing.
 *   - Conditions found on the device never cause out-of-bounds writes; they
 *     OR a bit into the caller's device status word (EP_STATUS_*), which the
 *     caller zeroes before ep_plan and reads after its own synchronisation.
 *     Rows that cannot be delivered are dropped and documented as such.
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the functions below are exported from the shared library. */
#define EP_API __attribute__((visibility("default")))

/* Return codes (host side). */
#define EP_OK 0
#define EP_ERR_INVALID_ARG (-1)     /* bad descriptor, size or null pointer */
#define EP_ERR_UNSUPPORTED (-2)     /* valid but outside the library's limits */
#define EP_ERR_DEVICE_MISMATCH (-3) /* a buffer is not on the stream's GPU */
#define EP_ERR_HIP (-4)             /* a HIP runtime call failed */

/* Device status bits, OR-ed into *status by ep_plan. */
#define EP_STATUS_BAD_EXPERT 1 /* an expert id outside [0, E): slot dropped */
#define EP_STATUS_CAPACITY 2   /* a rank would receive more than cap rows */
#define EP_STATUS_BAD_REGION 4 /* a KV region outside its pools: skipped */

/* Payload formats of the dispatched rows. */
#define EP_PAYLOAD_BF16 0     /* one plane: H bf16 values, 2H bytes per row */
#define EP_PAYLOAD_FP8_B128 1 /* plane 0: H OCP e4m3fn codes (H bytes);
                                 plane 1: H/128 fp32 block scales (H/32 B) */

/* Largest sizes the library accepts (EP_ERR_UNSUPPORTED beyond them). */
#define EP_MAX_EXPERTS 2048
#define EP_MAX_TOPK 64

/* Problem descriptor. cap_rows is the row capacity of every destination's
 * receive and grouped buffers; 0 selects the worst-case bound
 * N * T * max(R, E/N) ("Send and receive buffers"). Requirements:
 * all sizes > 0 except tokens >= 0, E % N == 0, H % 8 == 0 (bf16) or
 * H % 128 == 0 (fp8), R <= EP_MAX_TOPK, E <= EP_MAX_EXPERTS,
 * N * cap_rows < 2^31 and N * T * R * P < 2^26, where P is the number of
 * 1 KB pieces of a dispatch row (ceil(bytes / 1024) per plane, summed). */
typedef struct ep_desc {
    int32_t n_ranks;   /* N */
    int32_t tokens;    /* T, tokens per rank */
    int32_t hidden;    /* H */
    int32_t n_experts; /* E */
    int32_t topk;      /* R */
    int32_t payload;   /* EP_PAYLOAD_* */
    int64_t cap_rows;  /* rows per destination buffer; 0 = worst-case bound */
} ep_desc;

/* Device pointers into a plan workspace (see ep_plan for the contents). */
typedef struct ep_plan_view {
    int32_t *cnt;      /* [N][E]     rows source s sends to expert e */
    int32_t *send_off; /* [N][E+1]   exclusive prefix of cnt[s] over e */
    int32_t *send_pos; /* [N][T][R]  send-buffer row of each slot, or -1 */
    int32_t *recv_off; /* [N][N+1]   row at which rank d receives source s;
                                     recv_off[d][N] = rows d receives */
    int32_t *grp_off;  /* [N][L+1]   grouped-layout offset of local expert j */
    int32_t *grp_pos;  /* [N][T][R]  grouped row of each slot on its expert's
                                     rank, or -1 (bad id / over capacity) */
    int32_t *src_off;  /* [N][E]     rows sources 0..s-1 send to expert e */
    int32_t *comb_row; /* [N][T][R]  (e / L) * cap + grp_pos, or -1 */
    int32_t *grp_slot; /* [N*T*R]    slots in receive order: all delivered
                                     rows of rank 0 in grouped order, then
                                     rank 1, ...; slot id (s*T + t)*R + k;
                                     -1 after the last delivered row */
    int32_t *send_slot; /* [N][T*R]  slot id (s*T + t)*R + k that send row p
                                     of source s holds; -1 for p >= send_off[s][E] */
    int32_t *recv_rows; /* [N*T*R][2] receive order as row pairs: for the
                                     j-th delivered row (order of grp_slot),
                                     its send row s*T*R + send_pos and its
                                     grouped row d*cap + grp_pos; -1, -1 past
                                     the last delivered row */
    int32_t *send_seg;  /* [N][T*R]  for send row p < send_off[s][E] of s:
                                     d*T*R + i, where d is the destination
                                     rank and i = p - send_off[s][dL] the
                                     row's index in the segment s -> d;
                                     -1 for p >= send_off[s][E] */
    int32_t *win_list;  /* [N][nwin][W*R][2] or NULL: the windowed sender's
                                     work list, for sources of 4 to 32 MiB of
                                     token rows while all send buffers take at
                                     most 2 GiB. Window w of source s holds its
                                     tokens [w W, (w+1) W); its entries are
                                     the pairs (s*T*R + send_pos, s*T + t) of
                                     the window's slots in send-row order,
                                     then -1, -1. W is the largest power of two
                                     with W * (row bytes of all planes)
                                     <= 4 MiB; nwin = ceil(T / W). */
} ep_plan_view;

/* Worst-case receive rows N * T * max(R, E/N) ("Send and receive buffers");
 * -1 for an invalid descriptor. */
EP_API int64_t ep_recv_bound(const ep_desc *d);

/* Rows per destination buffer: cap_rows, or the bound when cap_rows == 0;
 * -1 for an invalid descriptor. */
EP_API int64_t ep_capacity(const ep_desc *d);

/* Number of payload planes (1 for bf16, 2 for fp8) and the bytes of one row
 * of plane p; 0 for an absent plane, -1 for an invalid descriptor. */
EP_API int ep_num_planes(const ep_desc *d);
EP_API int64_t ep_row_bytes(const ep_desc *d, int plane);

/* Bytes of the plan workspace for this descriptor (0 if invalid). The
 * caller allocates it on the device; it needs no initialisation. */
EP_API size_t ep_plan_bytes(const ep_desc *d);

/* Host-only: fill *v with pointers into plan_ws. No device access. */
EP_API int ep_plan_views(const ep_desc *d, void *plan_ws, ep_plan_view *v);

/* Plan ("Send and receive buffers"; counts and prefix sums of "Dispatch
 * and combine"). topk_idx: int32 [N][T][R] expert ids. Writes the whole
 * plan into plan_ws:
 *   cnt[s][e]       = #slots of s with expert e;
 *   send_off[s][e]  = sum_{e' < e} cnt[s][e']; rows for rank d are the
 *                     contiguous segment [send_off[s][dL], send_off[s][dL+L]);
 *   send_pos[s][t][k] = send_off[s][e] + #earlier slots (t', k') < (t, k) of
 *                     s with the same expert (stable: token, then choice);
 *   recv_off[d][s]  = sum_{s' < s} rows(s' -> d) (sources in rank order);
 *   grp_off[d][j]   = sum_{j' < j} sum_s cnt[s][dL + j'];
 *   src_off[s][e]   = sum_{s' < s} cnt[s'][e];
 *   grp_pos[s][t][k] = grp_off[d][j] + src_off[s][e] + send_pos - send_off[s][e]
 *                     (grouped order: local expert, source, token, choice);
 *   comb_row        = d * cap + grp_pos;
 *   grp_slot[j]     = the slot whose row is the j-th delivered row when the
 *                     ranks' grouped layouts are concatenated in rank order
 *                     (each truncated to cap rows); -1 for j past the end;
 *   send_slot[s][p] = the slot (s*T + t)*R + k with send_pos[s][t][k] = p
 *                     (the inverse of send_pos); -1 for p >= send_off[s][E];
 *   recv_rows[j]    = (s*T*R + send_pos, comb_row) of the slot grp_slot[j];
 *   send_seg[s][p]  = d*T*R + (p - send_off[s][dL]) for the rank d whose
 *                     segment holds send row p; -1 for p >= send_off[s][E];
 *   win_list        = the windowed sender's work list (see ep_plan_view),
 *                     written only when the descriptor has one.
 * Slots with an id outside [0, E) get -1 and set EP_STATUS_BAD_EXPERT; rows
 * with grp_pos >= cap get -1 and set EP_STATUS_CAPACITY. status: device
 * int32, bits OR-ed in. Deterministic: equal inputs give equal bytes. */
EP_API int ep_plan(const ep_desc *d, const int32_t *topk_idx, void *plan_ws,
            int32_t *status, hipStream_t stream);

/* Dispatch sender ("Dispatch and combine": the sender shuffles tokens into a
 * send buffer so that each peer takes one bulk write). For each plane p:
 * x[p] is [N][T][row_p], send[p] is [N][T*R][row_p];
 * send[p][s][send_pos[s][t][k]] = x[p][s][t] byte for byte. Each token row
 * is written R times. Slots with send_pos = -1 are skipped, and send rows
 * past send_off[s][E] are left untouched. plane 1 pointers must be NULL for
 * bf16. */
EP_API int ep_dispatch_pack(const ep_desc *d, const void *const x[2],
                     const void *plan_ws, void *const send[2],
                     hipStream_t stream);

/* Dispatch sender with block-fp8 quantisation fused in ("Evaluation":
 * block-scaled fp8 dispatch, bf16 combine). x: bf16 [N][T][H]; the
 * descriptor's payload must be EP_PAYLOAD_FP8_B128. Each token row is read
 * once and quantised per block of 128 values: scale = amax / 448 as a float
 * division (1 when amax is 0), code = OCP e4m3fn of x / scale (float
 * division), nearest even, clamped to +-448. NaN values are left out of
 * amax and a NaN quotient gets the NaN code 0x7F; an infinite value makes
 * its block's scale infinite, so its own code is 0x7F and the block's
 * finite values get (signed) zero codes. send[0] (codes, [N][T*R][H])
 * and send[1] (fp32 scales, [N][T*R][H/128]) receive the token's planes at
 * each of its R send positions, exactly as ep_dispatch_pack would place a
 * pre-quantised row. */
EP_API int ep_dispatch_pack_quant(const ep_desc *d, const uint16_t *x,
                                  const void *plan_ws, void *const send[2],
                                  hipStream_t stream);

/* The network write, materialised: for every pair (s, d) one bulk copy of
 * s's segment for d into d's receive buffer at recv_off[d][s].
 * recv[p] is [N][cap][row_p]; rows at or beyond cap are dropped. */
EP_API int ep_dispatch_transfer(const ep_desc *d, const void *const send[2],
                         const void *plan_ws, void *const recv[2],
                         hipStream_t stream);

/* Dispatch receiver on a materialised receive buffer: shuffle recv[p]
 * ([N][cap][row_p], as written by ep_dispatch_transfer) into the grouped
 * layout grouped[p] ([N][cap][row_p]; expert j of rank d owns rows
 * [grp_off[d][j], grp_off[d][j+1])). Under EP_STATUS_CAPACITY the receive
 * buffer lost the rows past cap in receive order (source, then segment
 * row), while the grouped layout keeps rows below cap in grouped order;
 * a grouped row below cap whose receive-buffer row was lost is written as
 * zeros. */
EP_API int ep_dispatch_unpack(const ep_desc *d, const void *const recv[2],
                       const void *plan_ws, void *const grouped[2],
                       hipStream_t stream);

/* Dispatch receiver with the transfer fused in: each destination pulls its
 * rows straight from the sources' send buffers (the pattern of intra-node
 * peer-mapped buffers) into the grouped layout:
 * grouped[p][e / L][grp_pos[s][t][k]] = send[p][s][send_pos[s][t][k]].
 * Same result as ep_dispatch_transfer followed by ep_dispatch_unpack when
 * no rank receives more than cap rows; under EP_STATUS_CAPACITY this path
 * delivers every row with grp_pos < cap, the staged path only those whose
 * receive-buffer row also fits (zeros in the others). */
EP_API int ep_dispatch_recv(const ep_desc *d, const void *const send[2],
                     const void *plan_ws, void *const grouped[2],
                     hipStream_t stream);

/* The whole dispatch in one call: ep_plan, ep_dispatch_pack and
 * ep_dispatch_recv, with identical results (plan_ws tables, send, grouped,
 * status). When a source's T R slots fit one plan chunk (4096), E <= 512 and
 * N <= 1024, it takes three launches instead of four: the send side of the plan, then
 * the sender with the count exchange ("Send and receive buffers") done by
 * extra blocks of the same launch, then the receiver. When, in addition, one
 * source's token rows take at most 4 MiB (the send-order sender) and all of
 * x at most 128 MiB, extra blocks of the plan launch read one dword of every
 * 128-byte line of x, so that the sender's first reads of each row find it
 * in the memory-side cache; x is only read. */
EP_API int ep_dispatch(const ep_desc *d, const int32_t *topk_idx,
                       const void *const x[2], void *plan_ws,
                       void *const send[2], void *const grouped[2],
                       int32_t *status, hipStream_t stream);

/* ep_dispatch with the quantising sender: ep_plan, ep_dispatch_pack_quant
 * and ep_dispatch_recv in one call (x: bf16 [N][T][H]; fp8 descriptor),
 * with the same results and the same launch saving, except that win_list
 * (the plain sender's work list) is not written. */
EP_API int ep_dispatch_quant(const ep_desc *d, const int32_t *topk_idx,
                             const uint16_t *x, void *plan_ws,
                             void *const send[2], void *const grouped[2],
                             int32_t *status, hipStream_t stream);

/* Split dispatch ("Dispatch and combine": dispatch is split into a sender
 * half and a receiver half so that other work can run between them; "Send
 * and receive buffers": each receiver keeps a small private region per
 * sender, which takes the first tokens together with the routing
 * information, before the counts have been exchanged).
 *
 * Sender half. Uses only each source rank's own data: the send side of the
 * plan (cnt[s], send_off[s], send_pos[s], send_slot[s], send_seg[s], as
 * ep_plan writes them; these rows are the routing information the source
 * publishes) and the pack, with
 * one change of destination: row i of the segment s -> d (the rows s sends
 * to the experts of rank d, which start at send_off[s][d L]) goes to
 * priv[p][(d N + s) P + i] when i < P = priv_rows, and to the send buffer
 * otherwise (those send rows are left unwritten).
 * priv: per plane [N][N][P][row_p] bytes; may be NULL when P == 0. P must be
 * in [0, T R]. status: as for ep_plan (bad expert ids). The receive-side
 * tables of plan_ws are not written. */
EP_API int ep_dispatch_send(const ep_desc *d, const int32_t *topk_idx,
                            const void *const x[2], void *plan_ws,
                            void *const send[2], void *const priv[2],
                            int32_t priv_rows, int32_t *status,
                            hipStream_t stream);

/* The sender half in two steps (ep_dispatch_send = send_plan, then
 * send_pack): send_plan writes cnt[s], send_off[s], send_pos[s],
 * send_slot[s], send_seg[s] (the routing information each source
 * publishes) and flags bad ids in status;
 * send_pack moves the rows (priv as for ep_dispatch_send). */
EP_API int ep_dispatch_send_plan(const ep_desc *d, const int32_t *topk_idx,
                                 void *plan_ws, int32_t *status,
                                 hipStream_t stream);
EP_API int ep_dispatch_send_pack(const ep_desc *d, const int32_t *topk_idx,
                                 const void *const x[2], const void *plan_ws,
                                 void *const send[2], void *const priv[2],
                                 int32_t priv_rows, hipStream_t stream);

/* Receiver half, after ep_dispatch_send on the same plan_ws (stream order
 * or an event). The exchange reads every source's published cnt row and
 * computes the receive side of the plan (src_off, recv_off, grp_off,
 * grp_pos, comb_row, grp_slot, recv_rows, capacity bit in status), then every
 * delivered row is moved into the grouped layout from wherever the sender
 * put it (private region or send buffer). Afterwards plan_ws and grouped
 * are identical to those of ep_plan, ep_dispatch_pack, ep_dispatch_recv. */
EP_API int ep_dispatch_recv_split(const ep_desc *d, const void *const send[2],
                                  void *const priv[2], int32_t priv_rows,
                                  void *plan_ws, void *const grouped[2],
                                  int32_t *status, hipStream_t stream);

/* The receiver half in two steps (ep_dispatch_recv_split = recv_plan, then
 * recv_pull). recv_plan needs only the counts the senders published
 * (after ep_dispatch_send_plan), not their rows, so it may run on another
 * stream while ep_dispatch_send_pack moves the data ("Send and receive
 * buffers": data movement need not wait for the count exchange);
 * recv_pull needs both. */
EP_API int ep_dispatch_recv_plan(const ep_desc *d, void *plan_ws,
                                 int32_t *status, hipStream_t stream);
EP_API int ep_dispatch_recv_pull(const ep_desc *d, const void *const send[2],
                                 void *const priv[2], int32_t priv_rows,
                                 const void *plan_ws, void *const grouped[2],
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * KV-block push ("vLLMにおける分離型推論のTTFTとTPOTを改善するプッシュ型KV転送",
 * sections 「実装の詳細」 and 「スレッドモデル」: the producer maps a
 * request's KV block ids to memory descriptors, merges contiguous blocks
 * into larger regions, writes them to every destination tensor-parallel
 * rank, and each producer rank's write carries a completion notification
 * that the consumer counts).
 *
 * Token i of a request lives at byte (blocks[i / block_tokens] *
 * block_tokens + i % block_tokens) * token_bytes of a pool, on each side
 * with its own block size and block table. A region moves `bytes` bytes
 * from src_off to dst_off; `first` is its offset in the request's byte
 * stream (the regions in token order, concatenated).
 * ---------------------------------------------------------------------- */
typedef struct ep_kv_region {
  int64_t src_off;
  int64_t dst_off;
  int64_t bytes;
  int64_t first;
} ep_kv_region;

/* Host only. Regions of one request of n_tokens tokens, in token order.
 * merge != 0: maximal runs (a region grows while the next token continues
 * on both sides); merge == 0: one region per piece of a source block that
 * lies in one destination block (the descriptors before merging).
 * token_bytes must be a positive multiple of 16; block sizes positive; ids
 * non-negative. Writes at most max_regions regions and returns their number,
 * or a negative EP_ERR_* code (EP_ERR_INVALID_ARG also when max_regions is
 * too small; n_tokens regions always suffice). */
EP_API int64_t ep_kv_plan(int64_t n_tokens, int64_t token_bytes,
                          int64_t src_block_tokens, const int32_t *src_blocks,
                          int64_t dst_block_tokens, const int32_t *dst_blocks,
                          int32_t merge, ep_kv_region *regions,
                          int64_t max_regions);

/* Device push of one request to `ranks` tensor-parallel ranks: rank r's
 * pools start at src_pool + r * src_rank_bytes and dst_pool +
 * r * dst_rank_bytes. regions: device array [n_regions] from ep_kv_plan;
 * total_bytes: their byte sum (a multiple of 16). notify: device int32 the
 * caller zeroes; each rank adds 1 once all its bytes are written (in stream
 * order after the copy), so the request has arrived when notify == ranks.
 * A region that does not fit its pools (or is not 16-byte aligned) is
 * skipped and sets EP_STATUS_BAD_REGION in status. */
EP_API int ep_kv_push(int32_t ranks, const ep_kv_region *regions,
                      int64_t n_regions, int64_t total_bytes,
                      const void *src_pool, int64_t src_rank_bytes,
                      void *dst_pool, int64_t dst_rank_bytes,
                      int32_t *notify, int32_t *status, hipStream_t stream);

/* The staged relay for comparison ("EFA の同じノード内の GPU 間通信: libfabric の shm と SAR", section 「SAR」:
 * segmentation and reassembly through bounce buffers of 32 KiB, at most 64
 * per message round, two copies per chunk): each rank's byte stream goes
 * round by round through `bounce` (device or pinned host memory of
 * bounce_slots * 32 KiB bytes, 1 <= bounce_slots <= 64), a sender copy into
 * the slots, then a receiver copy out of them. Same result and completion
 * counting as ep_kv_push. */
EP_API int ep_kv_push_staged(int32_t ranks, const ep_kv_region *regions,
                             int64_t n_regions, int64_t total_bytes,
                             const void *src_pool, int64_t src_rank_bytes,
                             void *dst_pool, int64_t dst_rank_bytes,
                             void *bounce, int32_t bounce_slots,
                             int32_t *notify, int32_t *status,
                             hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * ep_kv_push_staged with its bounce slots in the library's own device
 * memory instead of a caller buffer. That memory is one static array of
 * EP_KV_STATIC_SLOTS slots of 32 KiB (2 MiB) per GPU the library runs on,
 * held until the process ends. Arguments, result and completion counting
 * are those of ep_kv_push_staged without `bounce`; bounce_slots must be in
 * [1, EP_KV_STATIC_SLOTS], else EP_ERR_INVALID_ARG and nothing is enqueued.
 * The call allocates nothing. The slots need no initialisation: every round
 * writes the bytes it then reads. All calls on one GPU share its one array,
 * which keeps the last call's bytes: calls that overlap on one GPU (two
 * streams, or two threads without ordering between them) race and corrupt
 * each other's transfers, so such calls must be ordered by the caller. */
#define EP_KV_STATIC_SLOTS 64
EP_API int ep_kv_push_staged_static(int32_t ranks, const ep_kv_region *regions,
                                    int64_t n_regions, int64_t total_bytes,
                                    const void *src_pool, int64_t src_rank_bytes,
                                    void *dst_pool, int64_t dst_rank_bytes,
                                    int32_t bounce_slots, int32_t *notify,
                                    int32_t *status, hipStream_t stream);

/* Stand-in for the grouped GEMM (outside the method; used by tests and the
 * benchmark to produce expert outputs). expert_out is bf16 [N][cap][H].
 * bf16 payload: y = x when alpha == NULL, else y = bf16(x * alpha[e]) with a
 * float multiply; fp8 payload: y = bf16(decode(q) * scale of its 128-block).
 * Only delivered rows are written. */
EP_API int ep_expert_stub(const ep_desc *d, const void *const grouped[2],
                   const float *alpha, const void *plan_ws,
                   uint16_t *expert_out, hipStream_t stream);

/* Combine receiver ("Dispatch and combine": the weighted average of a
 * token's expert outputs, accumulated on its source rank).
 * expert_out: bf16 [N][cap][H]; weights: fp32 [N][T][R]; out: bf16 [N][T][H].
 * out[s][t][h] = bf16( sum_k w[s][t][k] * y[e_k / L][grp_pos[s][t][k]][h] ),
 * summed in fp32 in k order (fused multiply-add), rounded once to bf16
 * (nearest, ties to even). Dropped slots contribute nothing. */
EP_API int ep_combine(const ep_desc *d, const uint16_t *expert_out,
               const float *weights, const void *plan_ws, uint16_t *out,
               hipStream_t stream);

/* Combine with partial sums on the expert side ("Evaluation": accumulating
 * on the sender side of combine moves fewer bytes than accumulating on the
 * receiver only, at some cost in accuracy). For one token, the slots whose
 * experts sit on the same rank form a group; the first slot of a group is
 * its leader. Expert side: partial[s][t R + leader] = bf16( sum over the
 * group's slots, k order, of w_k * y_k ) in fp32 with fused multiply-adds
 * from 0, rounded once (nearest even); one row per (token, rank) pair is
 * what would travel back. Source side: out[s][t] = bf16( sum over the
 * token's leaders, k order, of partial ) in fp32 from 0, rounded once.
 * Dropped slots belong to no group; a token with none writes zeros.
 * partial: bf16 [N][T R][H], caller-owned scratch; only leader rows are
 * written. Results differ from ep_combine by the rounding of each partial
 * (one bf16 rounding per group). */
EP_API int ep_combine_presum(const ep_desc *d, const uint16_t *expert_out,
                             const float *weights, const void *plan_ws,
                             uint16_t *partial, uint16_t *out,
                             hipStream_t stream);

/* Copy `bytes` (a multiple of 16) from src to dst with the library's row
 * copy loop (non-temporal loads and stores, 7 KB per wave): a bandwidth
 * reference for measurements, not part of the method. Its non-temporal
 * accesses leave lines other kernels cached in place, so it does not serve
 * to evict the caches. */
EP_API int ep_probe_copy(void *dst, const void *src, size_t bytes,
                  hipStream_t stream);

/* Access-pattern probe: a bandwidth reference for measurements, not part of
 * the method. It moves data in the shapes the sender, receiver and combine
 * were chosen on. A launch walks `rows` rows in pieces of piece_bytes; each
 * wave handles one piece, consecutive waves consecutive pieces (or, with
 * waves > 0, that many waves walk the pieces grid-stride), 16 bytes per lane
 * at a time, with non-temporal stores. `table` (int32, fan_in entries per
 * walked row, or NULL) indexes a buffer of indexed_rows rows; entries
 * outside [0, indexed_rows) stand for row 0.
 *   EP_PROBE_COPY: dst row i = xor of fan_in (1, 2, 4 or 8) rows of src,
 *     rows table[i * fan_in + j] or, with table NULL, rows i + j * rows
 *     (fan_in = 1: a plain copy), loaded in_flight (1, 2, 4 or 8, dividing
 *     fan_in) rows at a time; src holds indexed_rows rows, dst `rows`;
 *   EP_PROBE_SCATTER: src row i written to dst rows table[i * fan_in + k]
 *     (with table NULL, rows i * fan_in + k), read once (in_flight = 1); src
 *     holds `rows` rows, dst indexed_rows;
 *   EP_PROBE_SCATTER_WIDE: the same from src rows of 2 * row_bytes, each
 *     16-byte output chunk c the xor of src chunks 2c and 2c + 1 (the 2:1
 *     narrowing of a bf16 -> one-byte sender);
 *   EP_PROBE_FILL: dst rows written with a pattern, src not read;
 *   EP_PROBE_READ: src rows (table[i] or i) read; dst (256 bytes) is
 *     written only where a lane's xor of its data equals 0x9e3779b9.
 *   Fill and read take fan_in = in_flight = 1.
 * Flags: EP_PROBE_NT_LOADS (non-temporal loads; else ordinary cached ones),
 * EP_PROBE_XCD (blocks renumbered as the sender's: XCD x takes the x-th
 * eighth of the pieces; one piece per wave only), EP_PROBE_ONE_WAVE
 * (workgroups of one wave instead of four, as the receiver launches).
 * Rows are row_bytes long, row-major; all buffers are caller-owned device
 * memory on the stream's GPU. row_bytes must be a multiple of piece_bytes,
 * piece_bytes of 1024. Returns EP_ERR_INVALID_ARG for a bad size, mode, flag
 * or buffer, EP_ERR_UNSUPPORTED beyond 2^31 pieces. */
#define EP_PROBE_COPY 0
#define EP_PROBE_FILL 1
#define EP_PROBE_READ 2
#define EP_PROBE_SCATTER 3
#define EP_PROBE_SCATTER_WIDE 4
#define EP_PROBE_NT_LOADS 1
#define EP_PROBE_XCD 2
#define EP_PROBE_ONE_WAVE 4
EP_API int ep_probe_pattern(void *dst, const void *src, const int32_t *table,
                            int64_t rows, int64_t indexed_rows, int64_t row_bytes,
                            int64_t piece_bytes, int fan_in, int in_flight, int mode,
                            int flags, int64_t waves, hipStream_t stream);

/* Text for a return code or status bit set; never NULL. */
EP_API const char *ep_status_string(int code);

/* Last host-side error message of the calling thread ("" if none). */
EP_API const char *ep_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
