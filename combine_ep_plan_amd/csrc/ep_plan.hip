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

#include "ep_device.hpp"
#include "ep_kernels.hpp"

namespace ep {
namespace {

// Exclusive prefix sum of a[0..n) in LDS, in place, by a block of
// kPlanThreads threads; writes the sum of all n values to *total (LDS).
// `scratch` holds kPlanThreads / 64 ints.
__device__ void block_exclusive_scan(int32_t* a, int n, int32_t* scratch, int32_t* total) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  constexpr int kWaves = kPlanThreads / kWave;
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int beg = tid * per;
  int local = 0;
  for (int q = 0; q < per; ++q)
    if (beg + q < n) local += a[beg + q];
  int inc = local;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < kWaves ? scratch[lane] : 0;
    int w = v;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int y = __shfl_up(w, off, kWave);
      if (lane >= off) w += y;
    }
    if (lane < kWaves) scratch[lane] = w - v;
    if (lane == kWaves - 1) *total = w;
  }
  __syncthreads();
  int run = scratch[wave] + (inc - local);
  for (int q = 0; q < per; ++q) {
    if (beg + q < n) {
      const int t = a[beg + q];
      a[beg + q] = run;
      run += t;
    }
  }
  __syncthreads();
}

// Ranks of the slots of chunk c of source s (ids in `src`, TR slots): for
// each of the kPlanSub sub-chunks of kPlanThreads slots, each wave ranks its
// 64 slots among equal ids (one ballot per id bit), and the waves' counts
// are combined by an exclusive prefix in LDS, continuing the running count
// of earlier sub-chunks. Returns, per sub-chunk, the slot's id (E for an
// invalid id or no slot) and its rank among the chunk's earlier slots with
// the same id; on return run[e] holds the chunk's count of id e.
// LDS: wcnt [kPlanThreads / 64][E + 1], run [E + 1].
__device__ __forceinline__ void chunk_ranks(const int32_t* __restrict__ src, int E, int64_t TR,
                                            int c, int32_t* wcnt, int32_t* run, int* e_of,
                                            int* rank_of, bool& bad) {
  constexpr int kWaves = kPlanThreads / kWave;
  const int Ep = E + 1;                 // bucket E collects invalid ids
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int nbits = 32 - __clz(E);      // bits of the values 0..E
  for (int q = tid; q < Ep; q += kPlanThreads) run[q] = 0;
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    e_of[sub] = E;
    rank_of[sub] = 0;
    const int64_t first = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads;
    if (first >= TR) continue;                                // block-uniform
    for (int q = tid; q < kWaves * Ep; q += kPlanThreads) wcnt[q] = 0;
    __syncthreads();
    const int64_t i = first + tid;
    const bool active = i < TR;
    int e = E;
    if (active) {
      e = src[i];
      if (e < 0 || e >= E) {
        e = E;
        bad = true;
      }
    }
    const uint64_t peers = match_key(e, nbits, active);
    const int rank = __popcll(peers & lanes_below());
    if (active && rank == 0) wcnt[wave * Ep + e] = __popcll(peers);
    __syncthreads();
    for (int q = tid; q < Ep; q += kPlanThreads) {
      int r = run[q];
      for (int w = 0; w < kWaves; ++w) {
        const int t = wcnt[w * Ep + q];
        wcnt[w * Ep + q] = r;
        r += t;
      }
      run[q] = r;
    }
    __syncthreads();
    e_of[sub] = e;
    if (active) rank_of[sub] = wcnt[wave * Ep + e] + rank;
    __syncthreads();
  }
}

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
  chunk_ranks(idx + (size_t)s * TR, E, TR, c, wcnt, run, e_of, rank_of, bad);
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

// Fetch this block's slots: expert ids and the per-slot value the previous
// launch left in send_pos (a rank inside the chunk, or a final position).
__device__ __forceinline__ void fetch_slots(const int32_t* __restrict__ idx,
                                            const int32_t* __restrict__ send_pos, int s, int c,
                                            int64_t TR, int* e_of, int* v_of) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    e_of[sub] = -1;
    v_of[sub] = -1;
    if (i < TR) {
      e_of[sub] = idx != nullptr ? idx[(size_t)s * TR + i] : 0;
      v_of[sub] = send_pos[(size_t)s * TR + i];
    }
  }
}

// The exchange: column sums over all sources of the per-expert counts. The
// sources are split across G thread groups (s2 = g, g + G, ...) so that all
// threads issue loads, then reduced through LDS. `count(s2, e)` is the
// count of expert e at source s2. On return (synced): gsc[e] = rows all
// sources send to e and sro[e], sros[e] = rows sources before s send to e.
template <typename Count>
__device__ __forceinline__ void column_sums(Count count, int N, int E, int s, int32_t* sro,
                                            int32_t* sros, int32_t* gsc, int32_t* part) {
  const int tid = threadIdx.x;
  const int G = E >= kPlanThreads ? 1 : kPlanThreads / E;
  int32_t* part_total = part;            // [G][E]
  int32_t* part_before = part + G * E;   // [G][E]
  for (int q = tid; q < G * E; q += kPlanThreads) {
    const int g = q / E, e = q % E;
    int total = 0, before = 0;
#pragma unroll 4
    for (int s2 = g; s2 < N; s2 += G) {
      const int v = count(s2, e);
      total += v;
      if (s2 < s) before += v;
    }
    part_total[q] = total;
    part_before[q] = before;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) {
    int total = 0, before = 0;
    for (int g = 0; g < G; ++g) {
      total += part_total[g * E + e];
      before += part_before[g * E + e];
    }
    sro[e] = before;
    sros[e] = before;
    gsc[e] = total;
  }
  __syncthreads();
}

// Receive side of the plan for the slots of block (c, s), from the sums of
// column_sums. within_of[sub] is the slot's index among the rows that s
// sends to its expert (negative: dropped slot). Writes src_off[s] and
// recv_off[.][s] (block c == 0), grp_off, the receive totals and the
// capacity flag (block (0, 0)), and grp_pos, comb_row and grp_slot of the
// block's slots; then clears the receive-order entries past the last
// delivered row (shared by all blocks).
__device__ void receive_tables(const int* e_of, const int* within_of, int s, int c, int N, int E,
                               int L, int64_t TR, int64_t cap, const PlanPtrs& p,
                               int32_t* status, int32_t* sro, int32_t* sros, int32_t* gsc,
                               int32_t* dstart, int32_t* scratch) {
  const int tid = threadIdx.x;
  if (c == 0)
    for (int e = tid; e < E; e += kPlanThreads) p.src_off[(size_t)s * E + e] = sro[e];
  block_exclusive_scan(sros, E, scratch, &sros[E]);
  block_exclusive_scan(gsc, E, scratch, &gsc[E]);
  // Receive order: the delivered rows of rank 0, then rank 1, ...
  for (int d = tid; d < N; d += kPlanThreads) {
    const int64_t total = gsc[(d + 1) * L] - gsc[d * L];
    dstart[d] = (int32_t)(total < cap ? total : cap);
  }
  __syncthreads();
  block_exclusive_scan(dstart, N, scratch, &dstart[N]);

  if (c == 0) {
    // Rank d receives source s after the rows of sources 0..s-1.
    for (int d = tid; d < N; d += kPlanThreads)
      p.recv_off[(size_t)d * (N + 1) + s] = sros[(d + 1) * L] - sros[d * L];
    if (s == 0) {
      for (int q = tid; q < N * (L + 1); q += kPlanThreads) {
        const int d = q / (L + 1), j = q % (L + 1);
        p.grp_off[q] = gsc[d * L + j] - gsc[d * L];
      }
      for (int d = tid; d < N; d += kPlanThreads) {
        const int total = gsc[(d + 1) * L] - gsc[d * L];
        p.recv_off[(size_t)d * (N + 1) + N] = total;
        if (total > cap) atomicOr(status, kStatusCapacity);
      }
    }
  }

#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    if (i >= TR) break;
    const size_t gi = (size_t)s * TR + i;
    const int e = e_of[sub];
    const int within = within_of[sub];
    if (e < 0 || e >= E || within < 0) {
      p.grp_pos[gi] = -1;
      p.comb_row[gi] = -1;
      continue;
    }
    const int d = e / L;
    const int64_t g = (int64_t)(gsc[e] - gsc[d * L]) + sro[e] + within;
    if (g < cap) {
      p.grp_pos[gi] = (int32_t)g;
      p.comb_row[gi] = (int32_t)((int64_t)d * cap + g);
      p.grp_slot[dstart[d] + g] = (int32_t)gi;
    } else {
      p.grp_pos[gi] = -1;
      p.comb_row[gi] = -1;
    }
  }
  const int64_t nblocks = (int64_t)gridDim.x * gridDim.y;
  const int64_t bl = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  for (int64_t j = dstart[N] + bl * kPlanThreads + tid; j < (int64_t)N * TR;
       j += nblocks * kPlanThreads)
    p.grp_slot[j] = -1;
}

// Per-source sums of the chunk counts: soff[e] = rows of s to e, pre[e] =
// rows of s to e in chunks before c.
__device__ __forceinline__ void source_sums(const int32_t* __restrict__ chunk_cnt, int s, int c,
                                            int E, int nchunks, int32_t* soff, int32_t* pre) {
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    const int32_t* cc = chunk_cnt + (size_t)s * nchunks * E + e;
    int sum = 0, part = 0;
    for (int c2 = 0; c2 < nchunks; ++c2) {
      const int v = cc[(size_t)c2 * E];
      sum += v;
      if (c2 < c) part += v;
    }
    soff[e] = sum;
    pre[e] = part;
  }
}

// Send side of the plan for the slots of block (c, s): cnt[s] and
// send_off[s] (block c == 0) and the final send positions. Returns each
// slot's index among the rows s sends to its expert (-1 for a bad id).
__device__ __forceinline__ void send_tables(const int* e_of, const int* rank_of, int s, int c,
                                            int E, int64_t TR, const PlanPtrs& p, int32_t* soff,
                                            const int32_t* pre, int32_t* scratch,
                                            int* within_of) {
  const int tid = threadIdx.x;
  if (c == 0)
    for (int e = tid; e < E; e += kPlanThreads) p.cnt[(size_t)s * E + e] = soff[e];
  block_exclusive_scan(soff, E, scratch, &soff[E]);
  if (c == 0)
    for (int e = tid; e <= E; e += kPlanThreads) p.send_off[(size_t)s * (E + 1) + e] = soff[e];
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    within_of[sub] = -1;
    if (i >= TR) continue;
    const int e = e_of[sub];
    if (e < 0 || e >= E) {
      p.send_pos[(size_t)s * TR + i] = -1;
      continue;
    }
    within_of[sub] = pre[e] + rank_of[sub];
    p.send_pos[(size_t)s * TR + i] = soff[e] + within_of[sub];
  }
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
  fetch_slots(idx, p.send_pos, s, c, TR, e_of, rank_of);
  const int32_t* cc = p.chunk_cnt;
  column_sums(
      [=](int s2, int e) {
        int sum = 0;
        for (int c2 = 0; c2 < nchunks; ++c2) sum += cc[((size_t)s2 * nchunks + c2) * E + e];
        return sum;
      },
      N, E, s, sro, sros, gsc, scratch + kPlanThreads / kWave);
  source_sums(p.chunk_cnt, s, c, E, nchunks, soff, pre);
  __syncthreads();
  send_tables(e_of, rank_of, s, c, E, TR, p, soff, pre, scratch, within_of);
  receive_tables(e_of, within_of, s, c, N, E, L, TR, cap, p, status, sro, sros, gsc, dstart,
                 scratch);
}

// Sender half of a split dispatch: the send side of the plan from the
// source's own chunk counts only (no data of any other rank).
__global__ __launch_bounds__(kPlanThreads) void plan_local_kernel(
    const int32_t* __restrict__ idx, int E, int64_t TR, int nchunks, PlanPtrs p) {
  extern __shared__ int32_t lds[];
  int32_t* soff = lds;               // [E+1]
  int32_t* pre = soff + (E + 1);     // [E]
  int32_t* scratch = pre + E;        // [kPlanThreads / 64]
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  int e_of[kPlanSub], rank_of[kPlanSub], within_of[kPlanSub];
  fetch_slots(idx, p.send_pos, s, c, TR, e_of, rank_of);
  source_sums(p.chunk_cnt, s, c, E, nchunks, soff, pre);
  __syncthreads();
  send_tables(e_of, rank_of, s, c, E, TR, p, soff, pre, scratch, within_of);
}

// Receiver half of a split dispatch: the exchange reads the counts every
// sender published (cnt rows) and the senders' own send offsets and
// positions; each slot's expert is the segment of send_off[s] its position
// falls in, so no routing ids are needed here.
__global__ __launch_bounds__(kPlanThreads) void plan_exchange_kernel(
    int N, int E, int L, int64_t TR, int64_t cap, PlanPtrs p, int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  int32_t* so = lds;                 // [E+1] send_off row of s
  int32_t* sro = so + (E + 1);       // [E]
  int32_t* sros = sro + E;           // [E+1]
  int32_t* gsc = sros + (E + 1);     // [E+1]
  int32_t* dstart = gsc + (E + 1);   // [N+1]
  int32_t* scratch = dstart + (N + 1);
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  int e_of[kPlanSub], pos_of[kPlanSub], within_of[kPlanSub];
  fetch_slots(nullptr, p.send_pos, s, c, TR, e_of, pos_of);
  for (int e = tid; e <= E; e += kPlanThreads) so[e] = p.send_off[(size_t)s * (E + 1) + e];
  const int32_t* cnt = p.cnt;
  column_sums([=](int s2, int e) { return cnt[(size_t)s2 * E + e]; }, N, E, s, sro, sros, gsc,
              scratch + kPlanThreads / kWave);
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int pos = pos_of[sub];
    e_of[sub] = -1;
    within_of[sub] = -1;
    if (pos < 0 || pos >= so[E]) continue;
    int lo = 0, hi = E - 1;  // largest e with so[e] <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (so[mid] <= pos) lo = mid; else hi = mid - 1;
    }
    e_of[sub] = lo;
    within_of[sub] = pos - so[lo];
  }
  receive_tables(e_of, within_of, s, c, N, E, L, TR, cap, p, status, sro, sros, gsc, dstart,
                 scratch);
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
  chunk_ranks(idx + (size_t)s * TR, E, TR, c, wcnt, run, e_of, rank_of, bad);
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
  send_tables(e_of, rank_of, s, c, E, TR, p, soff, pre, scratch, within_of);
  receive_tables(e_of, within_of, s, c, N, E, L, TR, cap, p, status, sro, sros, gsc, dstart,
                 scratch);
}

bool fused_plan_fits(const Dims& d) {
  return d.NTR <= kFusedPlanSlots && d.E <= 1024 && d.N <= 1024;
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
                        (const void*)plan_fused_kernel}) {
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

hipError_t launch_plan(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                       int32_t* status, hipStream_t stream) {
  hipError_t e = allow_large_lds();
  if (e != hipSuccess) return e;
  if (fused_plan_fits(d)) {
    hipLaunchKernelGGL(plan_fused_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                       lds_fused_bytes(d), stream, idx, d.N, d.E, d.L, d.TR, d.cap, p, status);
    return hipGetLastError();
  }
  e = launch_count(d, idx, p, status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_finalize_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                     lds_final_bytes(d), stream, idx, d.N, d.E, d.L, d.TR, d.nchunks, d.cap, p,
                     status);
  return hipGetLastError();
}

hipError_t launch_plan_local(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                             int32_t* status, hipStream_t stream) {
  hipError_t e = allow_large_lds();
  if (e != hipSuccess) return e;
  e = launch_count(d, idx, p, status, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_local_kernel, dim3(d.nchunks, d.N), dim3(kPlanThreads),
                     lds_final_bytes(d), stream, idx, d.E, d.TR, d.nchunks, p);
  return hipGetLastError();
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
