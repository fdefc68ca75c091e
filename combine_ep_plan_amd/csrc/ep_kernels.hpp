// Host-side launchers of the gfx950 kernels (one translation unit per
// kernel family). All sizes are validated by the C ABI layer before these
// are called; each launcher only shapes the grid and enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// Sizes derived from a validated descriptor.
struct Dims {
  int N, T, H, E, R, L, payload, planes;
  int64_t cap;       // rows per destination buffer
  int64_t TR;        // slots (and send rows) per source
  int64_t NT;        // tokens over all ranks
  int64_t NTR;       // slots over all ranks
  int64_t row[2];    // bytes per row of each payload plane (0 if absent)
  int nchunks;       // plan chunks per source
  int win;           // tokens per window of the windowed sender (0: not used)
  int nwin;          // windows per source
};

// Sender choice by the bytes of one source's token rows (all planes) and of
// all send buffers, from gfx950 measurements (see the senders): send order
// up to kGatherSourceBytes per source (the rows an XCD re-reads fit its 4 MB
// L2); windowed send order, windows of at most kGatherSourceBytes, up to
// kWindowSourceBytes per source while the send buffers take at most
// kWindowSendBytes; token order beyond.
constexpr int64_t kGatherSourceBytes = 4 << 20;
constexpr int64_t kWindowSourceBytes = 32 << 20;
constexpr int64_t kWindowSendBytes = (int64_t)2 << 30;

// Token rows the dispatch touches into the memory-side cache (MALL) at
// most, over all sources: beyond about half of its 256 MB they would evict
// each other before the sender reads them.
constexpr int64_t kTouchMaxBytes = (int64_t)128 << 20;

// Token rows the send-side plan launch touches for the sender (per plane:
// base pointer, or null, and one source's bytes).
struct RowTouch {
  const uint8_t* src[2];
  int64_t bytes[2];
};

// Plan workspace pointers (int32 arrays, see ep_plan_view).
struct PlanPtrs {
  int32_t *cnt, *send_off, *send_pos, *recv_off, *grp_off, *grp_pos, *src_off,
      *comb_row, *grp_slot, *chunk_cnt, *send_slot, *recv_rows, *send_seg, *win_list;
};

constexpr int kPlanThreads = 1024;
constexpr int kPlanSub = 4;                              // sub-chunks per block
constexpr int kPlanChunk = kPlanThreads * kPlanSub;      // slots per block
// Single-launch plan up to this many slots (N T R). Measured: 9.6 against
// 11.5 us (two launches) at 128 slots; 17.4 against 14.2 us at 32768 and
// 36.6 against 21.5 us at 65536, where every block histogramming all ids
// costs more than the second launch.
constexpr int64_t kFusedPlanSlots = 8192;

// with_window: also build the windowed sender's work list (when the
// descriptor has one); the quantising sender does not use it.
hipError_t launch_plan(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                       int32_t* status, hipStream_t stream, bool with_window = true);
// The windowed sender's work list (d.win > 0), from the send side of the plan.
hipError_t launch_window_list(const Dims& d, const PlanPtrs& p, hipStream_t stream);
// Split dispatch: the sender half's plan (no data of other ranks), the
// receiver half's exchange, and the two data movers with private regions of
// P rows per (destination, source) pair.
// touch (optional, the token rows the sender reads, per source): the
// send-side plan launch, when it is one launch (d.nchunks == 1), also reads
// one dword of every 128-byte line of them, so that the sender that follows
// finds them in the memory-side cache instead of HBM.
hipError_t launch_plan_local(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                             int32_t* status, hipStream_t stream, bool with_window = true,
                             const RowTouch* touch = nullptr);
hipError_t launch_plan_exchange(const Dims& d, const PlanPtrs& p, int32_t* status,
                                hipStream_t stream);
hipError_t launch_pack_split(const Dims& d, const int32_t* idx, const void* const x[2],
                             const PlanPtrs& p, void* const send[2], void* const priv[2], int P,
                             hipStream_t stream);
hipError_t launch_recv_split(const Dims& d, const void* const send[2], void* const priv[2], int P,
                             const PlanPtrs& p, void* const grouped[2], hipStream_t stream);
// Plan, pack and receive in one call (fewer launches when a source's slots
// fit one plan chunk; otherwise the three steps in turn).
hipError_t launch_dispatch(const Dims& d, const int32_t* idx, const void* const x[2],
                           const PlanPtrs& p, void* const send[2], void* const grouped[2],
                           int32_t* status, hipStream_t stream);
hipError_t launch_dispatch_quant(const Dims& d, const int32_t* idx, const uint16_t* x,
                                 const PlanPtrs& p, void* const send[2], void* const grouped[2],
                                 int32_t* status, hipStream_t stream);
// Whether the one-call dispatch can fold the count exchange into the sender
// launch, and the LDS bytes the exchange blocks need.
bool dispatch_fused_fits(const Dims& d);
size_t lds_exchange_bytes(const Dims& d, int threads_per_block);
hipError_t launch_pack(const Dims& d, const void* const x[2], const PlanPtrs& p,
                       void* const send[2], hipStream_t stream);
hipError_t launch_pack_quant(const Dims& d, const uint16_t* x, const PlanPtrs& p,
                             void* const send[2], hipStream_t stream);
hipError_t launch_recv(const Dims& d, const void* const send[2], const PlanPtrs& p,
                       void* const grouped[2], hipStream_t stream);
hipError_t launch_transfer(const Dims& d, const void* const send[2], const PlanPtrs& p,
                           void* const recv[2], hipStream_t stream);
hipError_t launch_unpack(const Dims& d, const void* const recv[2], const PlanPtrs& p,
                         void* const grouped[2], hipStream_t stream);
hipError_t launch_expert_stub(const Dims& d, const void* const grouped[2],
                              const float* alpha, const PlanPtrs& p, uint16_t* y,
                              hipStream_t stream);
hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* w,
                          const PlanPtrs& p, uint16_t* out, hipStream_t stream);
hipError_t launch_combine_presum(const Dims& d, const uint16_t* y, const float* w,
                                 const PlanPtrs& p, uint16_t* partial, uint16_t* out,
                                 hipStream_t stream);
// KV-block push (regions: device array of ep_kv_region).
int64_t kv_piece_bytes();
// The staged relay's bounce slots: 32 KiB each, at most 64 per round.
constexpr int64_t kKvSlotBytes = 32768;
constexpr int kKvStaticSlots = EP_KV_STATIC_SLOTS;
// Device address of the library's static bounce slots on `dev` (the current
// device), for the relay that allocates nothing.
hipError_t kv_static_bounce(int dev, void** out);
hipError_t launch_kv_push(int ranks, const ep_kv_region* reg, int64_t m, int64_t total,
                          const void* src, int64_t src_rank_bytes, void* dst,
                          int64_t dst_rank_bytes, int32_t* notify, int32_t* status,
                          hipStream_t stream);
hipError_t launch_kv_push_staged(int ranks, const ep_kv_region* reg, int64_t m, int64_t total,
                                 const void* src, int64_t src_rank_bytes, void* dst,
                                 int64_t dst_rank_bytes, void* bounce, int64_t round_bytes,
                                 int32_t* notify, int32_t* status, hipStream_t stream);
hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes,
                             hipStream_t stream);

}  // namespace ep
