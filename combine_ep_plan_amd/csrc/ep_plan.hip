// Plan kernels: per-(rank, expert) histogram, prefix sums, stable slot
// positions, and the one-GPU stand-in for the count exchange.
//
// Method: "Enabling trillion-parameter models on AWS EFA", section "Send
// and receive buffers" (counts are exchanged so that senders place rows
// contiguously per peer and receivers know each source's offset) and the
// dispatch timing figure of section "Dispatch and combine" (per-expert
// counts, then a running prefix sum gives the send offsets).
//
// The page counts with shared-memory atomics, which leave the order of rows
// inside an expert open. Here positions are stable (token, then choice) and
// deterministic: each wave ranks its 64 slots among equal expert ids with
// one ballot per id bit, and waves, sub-chunks and chunks are combined with
// exclusive prefix sums.
//
// Two launches (one, plan_fused_kernel, for small problems):
//   count:    grid (chunks, N). Per chunk of up to kPlanChunk slots of one
//             source: rank of each slot among earlier slots of the chunk with
//             the same expert (kept in send_pos), and the chunk's counts.
//   finalize: grid (chunks, N). Every block sums the chunk counts it needs
//             (all sources: the exchange), forms the prefix sums, writes the
//             tables once (chunk 0 blocks) and finishes its slots' positions.
#include <atomic>

#include "ep_plan_device.hpp"

namespace ep {
namespace {

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(
    const int32_t* __restrict__ idx, int E, int64_t TR, int nchunks,
    int32_t* __restrict__ lrank, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  constexpr int kWaves = kPlanThreads / kWave;
  int32_t* wcnt = lds;                        // [kWaves][E+1]
  int32_t* run = lds + kWaves * (E + 1);      // [E+1]
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  int e_of[kPlanSub], rank_of[kPlanSub];
  bool bad = false;
  chunk_ranks<kPlanThreads>(idx + (size_t)s * TR, E, TR, c, wcnt, run, e_of, rank_of, bad);
  int32_t* lr = lrank + (size_t)s * TR;
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    if (i < TR) lr[i] = rank_of[sub];
  }
  for (int q = tid; q < E; q += kPlanThreads)
    chunk_cnt[((size_t)s * nchunks + c) * E + q] = run[q];
  if (bad) atomicOr(status, kStatusBadExpert);
}

// The whole plan after the count launch: every block does the exchange (a
// redundant read of all sources' chunk counts), then both sides' tables.
__global__ __launch_bounds__(kPlanThreads) void plan_finalize_kernel(
    const int32_t* __restrict__ idx, int N, int E, int L, int64_t TR, int nchunks,
    int64_t cap, PlanPtrs p, int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  int32_t* soff = lds;               // [E+1] counts of s -> send offsets
  int32_t* pre = soff + (E + 1);     // [E]   rows of s in earlier chunks
  int32_t* sro = pre + E;            // [E]   rows earlier sources send to e
  int32_t* sros = sro + E;           // [E+1] prefix of sro over experts
  int32_t* gsc = sros + (E + 1);     // [E+1] prefix of column totals
  int32_t* dstart = gsc + (E + 1);   // [N+1] first receive-order row of rank d
  int32_t* scratch = dstart + (N + 1);  // [kPlanThreads / 64], then partial sums
  const int s = blockIdx.y;
  const int c = blockIdx.x;

  // Slots first, so that their latency overlaps the exchange.
  int e_of[kPlanSub], rank_of[kPlanSub], within_of[kPlanSub];
  fetch_slots<kPlanThreads>(idx, p.send_pos, s, c, TR, e_of, rank_of);
  const int32_t* cc = p.chunk_cnt;
  column_sums<kPlanThreads>(
      [=](int s2, int e) {
        int sum = 0;
        for (int c2 = 0; c2 < nchunks; ++c2) sum += cc[((size_t)s2 * nchunks + c2) * E + e];
        return sum;
      },
      N, E, s, sro, sros, gsc, scratch + kPlanThreads / kWave);
  source_sums<kPlanThreads>(p.chunk_cnt, s, c, E, nchunks, soff, pre);
  __syncthreads();
  send_tables<kPlanThreads>(e_of, rank_of, s, c, E, L, TR, p, soff, pre, scratch, within_of);
  receive_tables<kPlanThreads>(e_of, within_of, s, c, N, E, L, TR, cap, p, status, soff, sro,
                               sros, gsc,
                               dstart, scratch, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                               (int64_t)gridDim.x * gridDim.y);
}

// Sender half of a split dispatch: the send side of the plan from the
// source's own chunk counts only (no data of any other rank).
__global__ __launch_bounds__(kPlanThreads) void plan_local_kernel(
    const int32_t* __restrict__ idx, int E, int L, int64_t TR, int nchunks, PlanPtrs p) {
  extern __shared__ int32_t lds[];
  int32_t* soff = lds;               // [E+1]
  int32_t* pre = soff + (E + 1);     // [E]
  int32_t* scratch = pre + E;        // [kPlanThreads / 64]
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  int e_of[kPlanSub], rank_of[kPlanSub], within_of[kPlanSub];
  fetch_slots<kPlanThreads>(idx, p.send_pos, s, c, TR, e_of, rank_of);
  source_sums<kPlanThreads>(p.chunk_cnt, s, c, E, nchunks, soff, pre);
  __syncthreads();
  send_tables<kPlanThreads>(e_of, rank_of, s, c, E, L, TR, p, soff, pre, scratch, within_of);
}

// Receiver half of a split dispatch: the exchange reads the counts every
// sender published (cnt rows) and the senders' own send offsets and
// positions; each slot's expert is the segment of send_off[s] its position
// falls in, so no routing ids are needed here.
__global__ __launch_bounds__(kPlanThreads) void plan_exchange_kernel(
    int N, int E, int L, int64_t TR, int64_t cap, PlanPtrs p, int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  exchange_block<kPlanThreads>(blockIdx.y, blockIdx.x, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                               (int64_t)gridDim.x * gridDim.y, N, E, L, TR, cap, p, status, lds);
}

// The whole plan in one launch, for small problems (launch-bound: every
// block reads all N T R routing ids): block (c, s) ranks its chunk's
// slots, then builds the exchange directly from all sources' ids with LDS
// atomic counters (order-free totals, as the pages count), then writes both
// sides' tables like the finalize launch. Saves the count launch and the
// chunk-count round trip through memory.
__global__ __launch_bounds__(kPlanThreads) void plan_fused_kernel(
    const int32_t* __restrict__ idx, int N, int E, int L, int64_t TR, int64_t cap, PlanPtrs p,
    int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  constexpr int kWaves = kPlanThreads / kWave;
  int32_t* soff = lds;               // [E+1] rows of s to e -> send offsets
  int32_t* pre = soff + (E + 1);     // [E]   rows of s to e in earlier chunks
  int32_t* sro = pre + E;            // [E]   rows earlier sources send to e
  int32_t* sros = sro + E;           // [E+1]
  int32_t* gsc = sros + (E + 1);     // [E+1] rows all sources send to e
  int32_t* dstart = gsc + (E + 1);   // [N+1]
  int32_t* scratch = dstart + (N + 1);          // [kWaves]
  int32_t* wcnt = scratch + kWaves;             // [kWaves][E+1] (chunk ranks)
  int32_t* run = wcnt + kWaves * (E + 1);       // [E+1]
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPlanThreads) {
    soff[e] = 0;
    pre[e] = 0;
    sro[e] = 0;
    gsc[e] = 0;
  }
  int e_of[kPlanSub], rank_of[kPlanSub], within_of[kPlanSub];
  bool bad = false;
  chunk_ranks<kPlanThreads>(idx + (size_t)s * TR, E, TR, c, wcnt, run, e_of, rank_of, bad);
  if (bad) atomicOr(status, kStatusBadExpert);
  // The exchange: histograms over every source's ids.
  const int64_t mine = (int64_t)c * kPlanChunk;  // own slots before this chunk
  for (int s2 = 0; s2 < N; ++s2) {
    const int32_t* src = idx + (size_t)s2 * TR;
    for (int64_t j = tid; j < TR; j += kPlanThreads) {
      const int e = src[j];
      if (e < 0 || e >= E) continue;
      atomicAdd(&gsc[e], 1);
      if (s2 < s) {
        atomicAdd(&sro[e], 1);
      } else if (s2 == s) {
        atomicAdd(&soff[e], 1);
        if (j < mine) atomicAdd(&pre[e], 1);
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) sros[e] = sro[e];
  __syncthreads();
  send_tables<kPlanThreads>(e_of, rank_of, s, c, E, L, TR, p, soff, pre, scratch, within_of);
  receive_tables<kPlanThreads>(e_of, within_of, s, c, N, E, L, TR, cap, p, status, soff, sro,
                               sros, gsc,
                               dstart, scratch, (int64_t)blockIdx.y * gridDim.x + blockIdx.x,
                               (int64_t)gridDim.x * gridDim.y);
}

// Block x of source s touches lines [x * kTouchLines, (x + 1) * kTouchLines)
// of s's token rows in each plane: one dword of each 128-byte line with an
// ordinary load, which brings the line into the memory-side cache (MALL).
// The values are only held until they arrive. Two lines per thread spread
// the touch over about one block per CU at decode scale; with eight per
// thread (a quarter of the blocks) the flushed decode step took 340 against
// 330 us, with one 330 us.
constexpr int kTouchPerThread = 2;
constexpr int64_t kTouchLines = (int64_t)kPlanThreads * kTouchPerThread;

__device__ __forceinline__ void touch_rows(const RowTouch& t, int s, int x) {
  uint32_t acc = 0;
  for (int q = 0; q < 2; ++q) {
    if (t.src[q] == nullptr) continue;
    const int64_t bytes = t.bytes[q];
    const uint8_t* base = t.src[q] + (size_t)s * bytes;
    uint32_t v[kTouchPerThread];
#pragma unroll
    for (int k = 0; k < kTouchPerThread; ++k) {
      const int64_t line = (int64_t)x * kTouchLines + (int64_t)k * kPlanThreads + threadIdx.x;
      const int64_t off = line * 128 < bytes ? line * 128 : 0;
      v[k] = *(const uint32_t*)(base + off);
    }
#pragma unroll
    for (int k = 0; k < kTouchPerThread; ++k) acc ^= v[k];
  }
  asm volatile("" ::"v"(acc));
}

// Send side of the plan in one launch when a source's slots fit one chunk
// (T R <= kPlanChunk): ranks, counts and the scan together, so the send
// offsets and final positions need no chunk-count round trip. Grid
// (1 + touch blocks, N): block (0, s) plans source s; blocks (x > 0, s)
// touch s's token rows for the sender that follows (see RowTouch).
__global__ __launch_bounds__(kPlanThreads) void plan_count_local_kernel(
    const int32_t* __restrict__ idx, int E, int L, int64_t TR, PlanPtrs p,
    int32_t* __restrict__ status, RowTouch touch) {
  if (blockIdx.x > 0) {  // block-uniform
    touch_rows(touch, (int)blockIdx.y, (int)blockIdx.x - 1);
    return;
  }
  extern __shared__ int32_t lds[];
  constexpr int kWaves = kPlanThreads / kWave;
  int32_t* soff = lds;                        // [E+1]
  int32_t* pre = soff + (E + 1);              // [E] (zero: one chunk)
  int32_t* scratch = pre + E;                 // [kWaves]
  int32_t* wcnt = scratch + kWaves;           // [kWaves][E+1]
  int32_t* run = wcnt + kWaves * (E + 1);     // [E+1]
  const int s = blockIdx.y;
  int e_of[kPlanSub], rank_of[kPlanSub], within_of[kPlanSub];
  bool bad = false;
  chunk_ranks<kPlanThreads>(idx + (size_t)s * TR, E, TR, 0, wcnt, run, e_of, rank_of, bad);
  if (bad) atomicOr(status, kStatusBadExpert);
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    soff[e] = run[e];
    pre[e] = 0;
  }
  __syncthreads();
  send_tables<kPlanThreads>(e_of, rank_of, s, 0, E, L, TR, p, soff, pre, scratch, within_of);
}

// Work list of the windowed sender, block (w, s): the slots of source s's
// tokens [w W, (w+1) W) ordered by their send row. A window's rows of one
// expert are consecutive send rows (tokens ascend inside an expert's rows),
// so a slot's place in the list is the window's rows of the experts before
// its own (a histogram of the window, scanned) plus its send row minus the
// first send row of its expert in the window. The list has W R entries per
// window; the ones past the window's rows are (-1, -1).
__global__ __launch_bounds__(kPlanThreads) void window_list_kernel(int E, int T, int R, int W,
                                                                   int nwin, PlanPtrs p) {
  extern __shared__ int32_t lds[];
  int32_t* so = lds;                // [E+1] send_off[s]
  int32_t* cnt = so + (E + 1);      // [E+1] rows per expert, then their exclusive prefix
  int32_t* first = cnt + (E + 1);   // [E]   first send row of each expert in the window
  int32_t* scratch = first + E;     // [kPlanThreads / 64]
  const int s = blockIdx.y, w = blockIdx.x, tid = threadIdx.x;
  const int64_t TR = (int64_t)T * R;
  const int64_t lo = (int64_t)w * W * R;
  const int64_t hi = lo + (int64_t)W * R < TR ? lo + (int64_t)W * R : TR;
  for (int e = tid; e <= E; e += kPlanThreads) {
    so[e] = p.send_off[(size_t)s * (E + 1) + e];
    cnt[e] = 0;
    if (e < E) first[e] = INT32_MAX;
  }
  __syncthreads();
  auto expert_of = [&](int pos) {  // largest e with so[e] <= pos
    int a = 0, b = E - 1;
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (so[mid] <= pos) a = mid; else b = mid - 1;
    }
    return a;
  };
  for (int64_t i = lo + tid; i < hi; i += kPlanThreads) {
    const int pos = p.send_pos[(size_t)s * TR + i];
    if (pos < 0 || pos >= so[E]) continue;
    const int e = expert_of(pos);
    atomicAdd(&cnt[e], 1);
    atomicMin(&first[e], pos);
  }
  __syncthreads();
  block_exclusive_scan<kPlanThreads>(cnt, E, scratch, &cnt[E]);
  int2* list = (int2*)p.win_list + ((size_t)s * nwin + w) * W * R;
  for (int64_t i = lo + tid; i < hi; i += kPlanThreads) {
    const int pos = p.send_pos[(size_t)s * TR + i];
    if (pos < 0 || pos >= so[E]) continue;
    const int e = expert_of(pos);
    list[cnt[e] + (pos - first[e])] =
        make_int2((int32_t)((int64_t)s * TR + pos), (int32_t)((int64_t)s * T + i / R));
  }
  for (int64_t j = cnt[E] + tid; j < (int64_t)W * R; j += kPlanThreads) list[j] = make_int2(-1, -1);
}

size_t lds_window_bytes(const Dims& d) {
  return sizeof(int32_t) * ((size_t)3 * (d.E + 1) + kPlanThreads / kWave);
}

bool fused_plan_fits(const Dims& d) {
  return d.NTR <= kFusedPlanSlots && d.E <= 1024 && d.N <= 1024;
}

size_t lds_count_local_bytes(const Dims& d) {
  constexpr int kWaves = kPlanThreads / kWave;
  return sizeof(int32_t) * ((size_t)(kWaves + 3) * (d.E + 1) + kWaves);
}

size_t lds_fused_bytes(const Dims& d) {
  constexpr int kWaves = kPlanThreads / kWave;
  return sizeof(int32_t) * ((size_t)5 * (d.E + 1) + (d.N + 1) + kWaves +
                            (size_t)(kWaves + 1) * (d.E + 1));
}

// LDS bytes of the finalize and exchange launches (the larger of the two
// layouts) and of the count launch.
size_t lds_count_bytes(const Dims& d) {
  constexpr int kWaves = kPlanThreads / kWave;
  return sizeof(int32_t) * (size_t)(kWaves + 1) * (d.E + 1);
}
size_t lds_final_bytes(const Dims& d) {
  constexpr int kWaves = kPlanThreads / kWave;
  const int groups = d.E >= kPlanThreads ? 1 : kPlanThreads / d.E;
  return sizeof(int32_t) * ((size_t)5 * (d.E + 1) + (d.N + 1) + kWaves + (size_t)2 * groups * d.E);
}

// Kernels using more than 64 KB of LDS must opt in, once per device. The
// flags are atomics so that concurrent first calls from several threads are
// safe (the opt-in itself is idempotent).
hipError_t allow_large_lds() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::atomic<bool> done[64];
  const bool cached = dev >= 0 && dev < 64;
  if (cached && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  for (const void* f : {(const void*)plan_count_kernel, (const void*)plan_finalize_kernel,
                        (const void*)plan_local_kernel, (const void*)plan_exchange_kernel,
                        (const void*)plan_fused_kernel, (const void*)plan_count_local_kernel}) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
  }
  if (cached) done[dev].store(true, std::memory_order_release);
  return hipSuccess;
}

hipError_t launch_count(const Dims& d, const int32_t* idx, const PlanPtrs& p, int32_t* status,
                        hipStream_t stream) {
  hipLaunchKernelGGL(plan_count_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                     lds_count_bytes(d), stream, idx, d.E, d.TR, d.nchunks, p.send_pos,
                     p.chunk_cnt, status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_window_list(const Dims& d, const PlanPtrs& p, hipStream_t stream) {
  if (d.win <= 0 || d.NT == 0) return hipSuccess;
  hipLaunchKernelGGL(window_list_kernel, dim3(d.nwin, d.N), dim3(kPlanThreads),
                     lds_window_bytes(d), stream, d.E, d.T, d.R, d.win, d.nwin, p);
  return hipGetLastError();
}

hipError_t launch_plan(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                       int32_t* status, hipStream_t stream, bool with_window) {
  hipError_t e = allow_large_lds();
  if (e != hipSuccess) return e;
  if (fused_plan_fits(d)) {
    hipLaunchKernelGGL(plan_fused_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                       lds_fused_bytes(d), stream, idx, d.N, d.E, d.L, d.TR, d.cap, p, status);
  } else {
    e = launch_count(d, idx, p, status, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_finalize_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                       lds_final_bytes(d), stream, idx, d.N, d.E, d.L, d.TR, d.nchunks, d.cap, p,
                       status);
  }
  e = hipGetLastError();
  if (e != hipSuccess || !with_window) return e;
  return launch_window_list(d, p, stream);
}

hipError_t launch_plan_local(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                             int32_t* status, hipStream_t stream, bool with_window,
                             const RowTouch* touch) {
  hipError_t e = allow_large_lds();
  if (e != hipSuccess) return e;
  if (d.nchunks == 1) {
    RowTouch t{};
    int touch_blocks = 0;
    if (touch != nullptr && d.T > 0) {
      t = *touch;
      int64_t lines = 0;
      for (int q = 0; q < 2; ++q) {
        if (t.src[q] == nullptr) continue;
        const int64_t lq = (t.bytes[q] + 127) / 128;
        lines = lq > lines ? lq : lines;
      }
      touch_blocks = (int)((lines + kTouchLines - 1) / kTouchLines);
    }
    hipLaunchKernelGGL(plan_count_local_kernel, dim3(1 + touch_blocks, d.N), dim3(kPlanThreads),
                       lds_count_local_bytes(d), stream, idx, d.E, d.L, d.TR, p, status, t);
  } else {
    e = launch_count(d, idx, p, status, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(plan_local_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                       lds_final_bytes(d), stream, idx, d.E, d.L, d.TR, d.nchunks, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess || !with_window) return e;
  return launch_window_list(d, p, stream);
}

hipError_t launch_plan_exchange(const Dims& d, const PlanPtrs& p, int32_t* status,
                                hipStream_t stream) {
  hipError_t e = allow_large_lds();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_exchange_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                     lds_final_bytes(d), stream, d.N, d.E, d.L, d.TR, d.cap, p, status);
  return hipGetLastError();
}

}  // namespace ep
