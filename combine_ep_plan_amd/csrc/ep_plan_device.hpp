// Device side of the plan, shared by the plan kernels (1024-thread blocks)
// and the dispatch kernel that runs the count exchange beside the sender
// (256-thread blocks): TPB is the block size; every block covers one chunk
// of kPlanChunk slots of one source in kPlanChunk / TPB sub-chunks.
//
// Method: "Enabling trillion-parameter models on AWS EFA", sections "Send
// and receive buffers" and "Dispatch and combine" (see ep_plan.hip).
#pragma once

#include "ep_device.hpp"
#include "ep_kernels.hpp"

namespace ep {
namespace {

// Exclusive prefix sum of a[0..n) in LDS, in place, by a block of
// TPB threads; writes the sum of all n values to *total (LDS).
// `scratch` holds TPB / 64 ints.
template <int TPB>
__device__ void block_exclusive_scan(int32_t* a, int n, int32_t* scratch, int32_t* total) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  constexpr int kWaves = TPB / kWave;
  const int per = (n + TPB - 1) / TPB;
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
// each of the (kPlanChunk / TPB) sub-chunks of TPB slots, each wave ranks its
// 64 slots among equal ids (one ballot per id bit), and the waves' counts
// are combined by an exclusive prefix in LDS, continuing the running count
// of earlier sub-chunks. Returns, per sub-chunk, the slot's id (E for an
// invalid id or no slot) and its rank among the chunk's earlier slots with
// the same id; on return run[e] holds the chunk's count of id e.
// LDS: wcnt [TPB / 64][E + 1], run [E + 1].
template <int TPB>
__device__ __forceinline__ void chunk_ranks(const int32_t* __restrict__ src, int E, int64_t TR,
                                            int c, int32_t* wcnt, int32_t* run, int* e_of,
                                            int* rank_of, bool& bad) {
  constexpr int kWaves = TPB / kWave;
  const int Ep = E + 1;                 // bucket E collects invalid ids
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int nbits = 32 - __clz(E);      // bits of the values 0..E
  for (int q = tid; q < Ep; q += TPB) run[q] = 0;
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    e_of[sub] = E;
    rank_of[sub] = 0;
    const int64_t first = (int64_t)c * kPlanChunk + (int64_t)sub * TPB;
    if (first >= TR) continue;                                // block-uniform
    for (int q = tid; q < kWaves * Ep; q += TPB) wcnt[q] = 0;
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
    for (int q = tid; q < Ep; q += TPB) {
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

// Fetch this block's slots: expert ids and the per-slot value the previous
// launch left in send_pos (a rank inside the chunk, or a final position).
template <int TPB>
__device__ __forceinline__ void fetch_slots(const int32_t* __restrict__ idx,
                                            const int32_t* __restrict__ send_pos, int s, int c,
                                            int64_t TR, int* e_of, int* v_of) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * TPB + tid;
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
template <int TPB, typename Count>
__device__ __forceinline__ void column_sums(Count count, int N, int E, int s, int32_t* sro,
                                            int32_t* sros, int32_t* gsc, int32_t* part) {
  const int tid = threadIdx.x;
  const int G = E >= TPB ? 1 : TPB / E;
  int32_t* part_total = part;            // [G][E]
  int32_t* part_before = part + G * E;   // [G][E]
  for (int q = tid; q < G * E; q += TPB) {
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
  for (int e = tid; e < E; e += TPB) {
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

// Receive side of the plan for source s, in three parts, from the sums of
// column_sums (sro, sros, gsc).
//
// receive_prefix: src_off[s] and recv_off[.][s] (chunk c == 0), grp_off,
// the receive totals and the capacity flag (block (0, 0)). On return
// (synced) gsc[e] = rows all sources send to experts before e, sro[e] = rows
// sources before s send to e, dstart[d] = first receive-order row of rank d.
template <int TPB>
__device__ void receive_prefix(int s, int c, int N, int E, int L, int64_t cap, const PlanPtrs& p,
                               int32_t* status, int32_t* sro, int32_t* sros, int32_t* gsc,
                               int32_t* dstart, int32_t* scratch) {
  const int tid = threadIdx.x;
  if (c == 0)
    for (int e = tid; e < E; e += TPB) p.src_off[(size_t)s * E + e] = sro[e];
  block_exclusive_scan<TPB>(sros, E, scratch, &sros[E]);
  block_exclusive_scan<TPB>(gsc, E, scratch, &gsc[E]);
  // Receive order: the delivered rows of rank 0, then rank 1, ...
  for (int d = tid; d < N; d += TPB) {
    const int64_t total = gsc[(d + 1) * L] - gsc[d * L];
    dstart[d] = (int32_t)(total < cap ? total : cap);
  }
  __syncthreads();
  block_exclusive_scan<TPB>(dstart, N, scratch, &dstart[N]);

  if (c == 0) {
    // Rank d receives source s after the rows of sources 0..s-1.
    for (int d = tid; d < N; d += TPB)
      p.recv_off[(size_t)d * (N + 1) + s] = sros[(d + 1) * L] - sros[d * L];
    if (s == 0) {
      for (int q = tid; q < N * (L + 1); q += TPB) {
        const int d = q / (L + 1), j = q % (L + 1);
        p.grp_off[q] = gsc[d * L + j] - gsc[d * L];
      }
      for (int d = tid; d < N; d += TPB) {
        const int total = gsc[(d + 1) * L] - gsc[d * L];
        p.recv_off[(size_t)d * (N + 1) + N] = total;
        if (total > cap) atomicOr(status, kStatusCapacity);
      }
    }
  }
}

// receive_slot: grp_pos, comb_row, grp_slot and recv_rows of slot i of s,
// whose expert is e and which is the within-th row s sends to e (e outside
// [0, E) or within < 0: a dropped slot). so: send_off[s].
__device__ __forceinline__ void receive_slot(int64_t i, int e, int within, int s, int E, int L,
                                             int64_t TR, int64_t cap, const PlanPtrs& p,
                                             const int32_t* so, const int32_t* sro,
                                             const int32_t* gsc, const int32_t* dstart) {
  const size_t gi = (size_t)s * TR + i;
  if (e < 0 || e >= E || within < 0) {
    p.grp_pos[gi] = -1;
    p.comb_row[gi] = -1;
    return;
  }
  const int d = e / L;
  const int64_t g = (int64_t)(gsc[e] - gsc[d * L]) + sro[e] + within;
  if (g < cap) {
    p.grp_pos[gi] = (int32_t)g;
    p.comb_row[gi] = (int32_t)((int64_t)d * cap + g);
    p.grp_slot[dstart[d] + g] = (int32_t)gi;
    ((int2*)p.recv_rows)[dstart[d] + g] =
        make_int2((int32_t)((int64_t)s * TR + so[e] + within), (int32_t)((int64_t)d * cap + g));
  } else {
    p.grp_pos[gi] = -1;
    p.comb_row[gi] = -1;
  }
}

// receive_clear: the receive-order entries past the last delivered row,
// shared by all nblocks blocks doing this work (this one is bl).
template <int TPB>
__device__ __forceinline__ void receive_clear(int N, int64_t TR, const PlanPtrs& p,
                                              const int32_t* dstart, int64_t bl, int64_t nblocks) {
  for (int64_t j = dstart[N] + bl * TPB + threadIdx.x; j < (int64_t)N * TR; j += nblocks * TPB) {
    p.grp_slot[j] = -1;
    ((int2*)p.recv_rows)[j] = make_int2(-1, -1);
  }
}

// All three for the slots of block (c, s), whose experts and within-expert
// indices the caller holds (within_of[sub] < 0: dropped slot).
template <int TPB>
__device__ void receive_tables(const int* e_of, const int* within_of, int s, int c, int N, int E,
                               int L, int64_t TR, int64_t cap, const PlanPtrs& p,
                               int32_t* status, const int32_t* so, int32_t* sro, int32_t* sros,
                               int32_t* gsc, int32_t* dstart, int32_t* scratch, int64_t bl,
                               int64_t nblocks) {
  receive_prefix<TPB>(s, c, N, E, L, cap, p, status, sro, sros, gsc, dstart, scratch);
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * TPB + threadIdx.x;
    if (i >= TR) break;
    receive_slot(i, e_of[sub], within_of[sub], s, E, L, TR, cap, p, so, sro, gsc, dstart);
  }
  receive_clear<TPB>(N, TR, p, dstart, bl, nblocks);
}

// Per-source sums of the chunk counts: soff[e] = rows of s to e, pre[e] =
// rows of s to e in chunks before c.
template <int TPB>
__device__ __forceinline__ void source_sums(const int32_t* __restrict__ chunk_cnt, int s, int c,
                                            int E, int nchunks, int32_t* soff, int32_t* pre) {
  for (int e = threadIdx.x; e < E; e += TPB) {
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
// send_off[s] (block c == 0), the final send positions and their inverse
// (send_slot: the slot each send row holds, -1 for the rows past the last
// one s fills), and send_seg: for each send row, its destination rank d and
// index i inside the segment s -> d, as d * T R + i (-1 past the rows s
// fills). Returns each slot's
// index among the rows s sends to its expert (-1 for a bad id).
template <int TPB>
__device__ __forceinline__ void send_tables(const int* e_of, const int* rank_of, int s, int c,
                                            int E, int L, int64_t TR, const PlanPtrs& p,
                                            int32_t* soff, const int32_t* pre, int32_t* scratch,
                                            int* within_of) {
  const int tid = threadIdx.x;
  if (c == 0)
    for (int e = tid; e < E; e += TPB) p.cnt[(size_t)s * E + e] = soff[e];
  block_exclusive_scan<TPB>(soff, E, scratch, &soff[E]);
  if (c == 0) {
    for (int e = tid; e <= E; e += TPB) p.send_off[(size_t)s * (E + 1) + e] = soff[e];
    for (int64_t j = soff[E] + tid; j < TR; j += TPB) {
      p.send_slot[(size_t)s * TR + j] = -1;
      p.send_seg[(size_t)s * TR + j] = -1;
    }
  }
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * TPB + tid;
    within_of[sub] = -1;
    if (i >= TR) continue;
    const int e = e_of[sub];
    if (e < 0 || e >= E) {
      p.send_pos[(size_t)s * TR + i] = -1;
      continue;
    }
    within_of[sub] = pre[e] + rank_of[sub];
    const int pos = soff[e] + within_of[sub];
    const int d = e / L;
    p.send_pos[(size_t)s * TR + i] = pos;
    p.send_slot[(size_t)s * TR + pos] = (int32_t)((size_t)s * TR + i);
    p.send_seg[(size_t)s * TR + pos] = (int32_t)(d * TR + (pos - soff[d * L]));
  }
}


// The receive side of the plan for the slots of block (c, s) from the
// counts every sender published (cnt rows) and the senders' own send
// offsets and positions; each slot's expert is the segment of send_off[s]
// its position falls in, so no routing ids are needed. bl / nblocks: this
// block's index among the blocks doing this work, and their number.
template <int TPB>
__device__ void exchange_block(int s, int c, int64_t bl, int64_t nblocks, int N, int E, int L,
                               int64_t TR, int64_t cap, const PlanPtrs& p,
                               int32_t* __restrict__ status, int32_t* lds) {
  int32_t* so = lds;                 // [E+1] send_off row of s
  int32_t* sro = so + (E + 1);       // [E]
  int32_t* sros = sro + E;           // [E+1]
  int32_t* gsc = sros + (E + 1);     // [E+1]
  int32_t* dstart = gsc + (E + 1);   // [N+1]
  int32_t* scratch = dstart + (N + 1);
  const int tid = threadIdx.x;
  // The slots' send positions first, so that their latency overlaps the
  // exchange; only the positions are held across it (the expert and the
  // within-expert index are derived afterwards, which keeps the register
  // count low for the sender launches this block shares).
  int pos_of[kPlanChunk / TPB];
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * TPB + tid;
    pos_of[sub] = i < TR ? p.send_pos[(size_t)s * TR + i] : -1;
  }
  for (int e = tid; e <= E; e += TPB) so[e] = p.send_off[(size_t)s * (E + 1) + e];
  const int32_t* cnt = p.cnt;
  column_sums<TPB>([=](int s2, int e) { return cnt[(size_t)s2 * E + e]; }, N, E, s, sro, sros, gsc,
              scratch + TPB / kWave);
  receive_prefix<TPB>(s, c, N, E, L, cap, p, status, sro, sros, gsc, dstart, scratch);
  // The expert of a slot is the segment of send_off[s] its position falls in.
#pragma unroll
  for (int sub = 0; sub < (kPlanChunk / TPB); ++sub) {
    const int64_t i = (int64_t)c * kPlanChunk + (int64_t)sub * TPB + tid;
    if (i >= TR) break;
    const int pos = pos_of[sub];
    int e = -1, within = -1;
    if (pos >= 0 && pos < so[E]) {
      int lo = 0, hi = E - 1;  // largest e with so[e] <= pos
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (so[mid] <= pos) lo = mid; else hi = mid - 1;
      }
      e = lo;
      within = pos - so[lo];
    }
    receive_slot(i, e, within, s, E, L, TR, cap, p, so, sro, gsc, dstart);
  }
  receive_clear<TPB>(N, TR, p, dstart, bl, nblocks);
}

}  // namespace
}  // namespace ep
