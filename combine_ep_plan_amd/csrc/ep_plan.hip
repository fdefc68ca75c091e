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
// Two launches:
//   count:    grid (chunks, N). Per chunk of up to kPlanChunk slots of one
//             source: rank of each slot among earlier slots of the chunk with
//             the same expert (kept in send_pos), and the chunk's counts.
//   finalize: grid (chunks, N). Every block sums the chunk counts it needs
//             (all sources: the exchange), forms the prefix sums, writes the
//             tables once (chunk 0 blocks) and finishes its slots' positions.
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

__global__ __launch_bounds__(kPlanThreads) void plan_count_kernel(
    const int32_t* __restrict__ idx, int E, int64_t TR, int nchunks,
    int32_t* __restrict__ lrank, int32_t* __restrict__ chunk_cnt,
    int32_t* __restrict__ status) {
  extern __shared__ int32_t lds[];
  constexpr int kWaves = kPlanThreads / kWave;
  const int Ep = E + 1;                 // bucket E collects invalid ids
  int32_t* wcnt = lds;                  // [kWaves][Ep]
  int32_t* run = lds + kWaves * Ep;     // [Ep] running count over sub-chunks
  const int s = blockIdx.y;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int nbits = 32 - __clz(E);      // bits of the values 0..E
  const int32_t* src = idx + (size_t)s * TR;
  int32_t* lr = lrank + (size_t)s * TR;
  bool bad = false;

  for (int q = tid; q < Ep; q += kPlanThreads) run[q] = 0;
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t first = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads;
    if (first >= TR) break;                                   // block-uniform
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
    // Per expert: exclusive prefix over the waves, continuing the running
    // count of earlier sub-chunks.
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
    if (active) lr[i] = wcnt[wave * Ep + e] + rank;
    __syncthreads();
  }
  for (int q = tid; q < E; q += kPlanThreads)
    chunk_cnt[((size_t)s * nchunks + c) * E + q] = run[q];
  if (bad) atomicOr(status, kStatusBadExpert);
}

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
  const int tid = threadIdx.x;

  // This block's slots: expert ids and the ranks left by the count kernel,
  // fetched first so that their latency overlaps the exchange below.
  const int32_t* src = idx + (size_t)s * TR;
  int e_of[kPlanSub], rank_of[kPlanSub];
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    e_of[sub] = -1;
    rank_of[sub] = 0;
    if (i < TR) {
      e_of[sub] = src[i];
      rank_of[sub] = p.send_pos[(size_t)s * TR + i];
    }
  }

  // The exchange: every block reads the counts of all sources. The column
  // sums over sources are split across G thread groups (sources s2 = g,
  // g + G, ...) so that all threads issue loads, then reduced through LDS.
  const int G = E >= kPlanThreads ? 1 : kPlanThreads / E;
  int32_t* part_total = scratch + kPlanThreads / kWave;  // [G][E]
  int32_t* part_before = part_total + G * E;             // [G][E]
  for (int q = tid; q < G * E; q += kPlanThreads) {
    const int g = q / E, e = q % E;
    int total = 0, before = 0;
#pragma unroll 4
    for (int s2 = g; s2 < N; s2 += G) {
      const int32_t* cc = p.chunk_cnt + (size_t)s2 * nchunks * E + e;
      int sum = 0, part = 0;
      for (int c2 = 0; c2 < nchunks; ++c2) {
        const int v = cc[(size_t)c2 * E];
        sum += v;
        if (c2 < c) part += v;
      }
      total += sum;
      if (s2 < s) before += sum;
      if (s2 == s) {
        soff[e] = sum;
        pre[e] = part;
      }
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
  if (c == 0) {
    for (int e = tid; e < E; e += kPlanThreads) {
      p.cnt[(size_t)s * E + e] = soff[e];
      p.src_off[(size_t)s * E + e] = sro[e];
    }
  }
  block_exclusive_scan(soff, E, scratch, &soff[E]);
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
    for (int e = tid; e <= E; e += kPlanThreads) p.send_off[(size_t)s * (E + 1) + e] = soff[e];
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

  // Final positions of this block's slots.
#pragma unroll
  for (int sub = 0; sub < kPlanSub; ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * kPlanThreads + tid;
    if (i >= TR) break;
    const size_t gi = (size_t)s * TR + i;
    const int e = e_of[sub];
    if (e < 0 || e >= E) {
      p.send_pos[gi] = -1;
      p.grp_pos[gi] = -1;
      p.comb_row[gi] = -1;
      continue;
    }
    const int within = pre[e] + rank_of[sub];
    p.send_pos[gi] = soff[e] + within;
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
  // Receive-order entries past the last delivered row, shared by all blocks.
  const int64_t nblocks = (int64_t)gridDim.x * gridDim.y;
  const int64_t bl = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  for (int64_t j = dstart[N] + bl * kPlanThreads + tid; j < (int64_t)N * TR;
       j += nblocks * kPlanThreads)
    p.grp_slot[j] = -1;
}

}  // namespace

hipError_t launch_plan(const Dims& d, const int32_t* idx, const PlanPtrs& p,
                       int32_t* status, hipStream_t stream) {
  constexpr int kWaves = kPlanThreads / kWave;
  const size_t lds_count = sizeof(int32_t) * (size_t)(kWaves + 1) * (d.E + 1);
  const int groups = d.E >= kPlanThreads ? 1 : kPlanThreads / d.E;
  const size_t lds_final = sizeof(int32_t) * ((size_t)5 * (d.E + 1) + (d.N + 1) + kWaves +
                                              (size_t)2 * groups * d.E);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)plan_count_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)plan_finalize_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(d.nchunks, d.N);
  hipLaunchKernelGGL(plan_count_kernel, grid, dim3(kPlanThreads), lds_count, stream, idx, d.E,
                     d.TR, d.nchunks, p.send_pos, p.chunk_cnt, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(plan_finalize_kernel, grid, dim3(kPlanThreads), lds_final, stream, idx, d.N,
                     d.E, d.L, d.TR, d.nchunks, d.cap, p, status);
  return hipGetLastError();
}

}  // namespace ep
