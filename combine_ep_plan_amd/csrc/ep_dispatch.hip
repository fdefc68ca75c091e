// Dispatch data movement: the senders (plain, split with private regions,
// and with the count exchange folded in), the per-pair transfer, the
// receiver unpack, and the receivers with the transfer fused in (pull).
//
// Method: "Enabling trillion-parameter models on AWS EFA", section
// "Dispatch and combine": the sender shuffles tokens into a send buffer laid
// out so that each peer takes one bulk write; the receiver shuffles its
// receive buffer into the grouped-GEMM input; within a node, buffers mapped
// into the peers let a rank pull tokens directly.
//
// Rows move as opaque bytes; lane l of a wave moves 16-byte chunks l, l+64,
// ... and all chunks a wave holds are loaded before the first store. Row
// indices are wave-uniform and live in scalar registers. Two shapes:
//   - 1 KB pieces in output order (the sender in send order, the receiver in
//     receive order, the staged transfer and unpack): consecutive waves
//     write consecutive 1 KB pieces, so the stores advance through memory as
//     one front; measured on gfx950 this beats whole rows per wave for
//     store-heavy copies (a fill writes 6.8 TB/s with 1 KB per wave against
//     5.3 TB/s with 14 KB). Each wave needs one or two table loads to find
//     its rows.
//   - whole rows per token pair (the token-order senders, for sources of
//     more than 32 MiB of token rows or send buffers of more than 2 GiB; in
//     between, the send-order sender walks windows of tokens): one wave
//     loads two token rows and writes each to its R send rows.
#include "ep_device.hpp"
#include "ep_kernels.hpp"
#include "ep_plan_device.hpp"

namespace ep {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
// The receiver (and the staged transfer and unpack, the same 1 KB-piece
// copies) run one wave per workgroup. Measured on gfx950 against four (same
// pieces, same order, 20 back-to-back launches): 143.5 against 148.5 us at
// decode scale, 282 against 302 us on the all-to-one workload; transfer +
// unpack at decode 284-289 against 295-297 us.
// The finer grain lets the dispatcher keep every CU's wave slots filled
// with independent 1 KB pieces. The senders keep four-wave groups: with one
// wave per group the send-order sender took 102-104 against 74-76 us at
// decode scale (two waves: the same as four), and the count exchange that
// runs in its first blocks needs 256 threads.
constexpr int kRecvWaves = 1;
constexpr int kRecvBlock = kRecvWaves * kWave;
constexpr int kSegV = 7;   // 16-byte chunks per lane in a row segment
constexpr int kSeg = kWave * kSegV;  // 16-byte chunks per segment (7 KB)
// The senders read token rows with ordinary (cached) loads: measured on
// gfx950 against non-temporal loads, pack took 405 vs 466 us at prefill
// scale and 185 vs 211 us on the all-to-one workload, and was neutral at
// decode scale. Every other copy reads non-temporally (its reads measured
// faster that way: the receiver 157 vs 169 us at decode scale; with one-wave
// groups 142-148 vs 158-161 us, and cached reads of the send rows also
// evicted the token rows from the memory-side cache, so the next step's
// sender took 97-103 instead of 73 us).
constexpr bool kPackNtLoads = false;

struct Planes {
  const uint8_t* src[2];
  uint8_t* dst[2];
  int64_t row[2];
  int planes;
};

__device__ __forceinline__ int wave_index() {
  return wave_uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
}

// Sender: one wave per pair of tokens. Both token rows are loaded (up to
// 28 KB in flight per wave), then each is written to its R send slots. Unlike
// the plain copies, pack is store-heavy (R stores per load) and measured
// fastest with whole 14 KB rows per wave (14 chunks per lane) and one wave
// per token pair: 99.5 us against 105.5 us for 7 KB segments at decode
// scale. send rows of source s start at s * T * R.
template <int V>
__device__ __forceinline__ void pack_stores(const RowRegs<V>& r, uint8_t* dst0, const int32_t* sp,
                                            int R, int TR, size_t row, int base, int n16) {
  for (int k = 0; k < R; ++k) {
    const int p = sp[k];
    if (p < 0 || p >= TR) continue;
    store_row16(r, (u32x4*)(dst0 + (size_t)p * row), base, n16);
  }
}

// One plane of the token pair tok0, tok0 + 1 (the second may not exist).
template <int V>
__device__ __forceinline__ void pack_plane(const uint8_t* x, uint8_t* send,
                                           const int32_t* __restrict__ send_pos, int tok0,
                                           bool two, int T, int R, size_t row) {
  const int TR = T * R;
  const int n16 = (int)(row >> 4);
  for (int base = 0; base < n16; base += kWave * V) {
    RowRegs<V> r0, r1;
    load_row16<V, kPackNtLoads>(r0, (const u32x4*)(x + (size_t)tok0 * row), base, n16);
    if (two) load_row16<V, kPackNtLoads>(r1, (const u32x4*)(x + (size_t)(tok0 + 1) * row), base, n16);
    pack_stores(r0, send + (size_t)(tok0 / T) * TR * row, send_pos + (size_t)tok0 * R, R, TR,
                row, base, n16);
    if (two)
      pack_stores(r1, send + (size_t)((tok0 + 1) / T) * TR * row,
                  send_pos + (size_t)(tok0 + 1) * R, R, TR, row, base, n16);
  }
}

__global__ __launch_bounds__(kBlock) void pack_kernel(Planes pl, const int32_t* __restrict__ send_pos,
                                                      int NT, int T, int R) {
  const int tok0 = 2 * wave_index();
  if (tok0 >= NT) return;
  const bool two = tok0 + 1 < NT;
  const int TR = T * R;
  for (int q = 0; q < pl.planes; ++q) {
    const size_t row = (size_t)pl.row[q];
    if ((row & 15) == 0) {
      const int n16 = (int)(row >> 4);
      if (n16 > kSeg)
        pack_plane<2 * kSegV>(pl.src[q], pl.dst[q], send_pos, tok0, two, T, R, row);
      else if (n16 > kWave)
        pack_plane<kSegV>(pl.src[q], pl.dst[q], send_pos, tok0, two, T, R, row);
      else
        pack_plane<1>(pl.src[q], pl.dst[q], send_pos, tok0, two, T, R, row);
    } else {
      for (int u = 0; u < (two ? 2 : 1); ++u) {
        const int tok = tok0 + u;
        const int32_t* sp = send_pos + (size_t)tok * R;
        uint8_t* dst0 = pl.dst[q] + (size_t)(tok / T) * TR * row;
        for (int k = 0; k < R; ++k) {
          const int p = sp[k];
          if (p < 0 || p >= TR) continue;
          copy_row4((const uint32_t*)(pl.src[q] + (size_t)tok * row),
                    (uint32_t*)(dst0 + (size_t)p * row), (int64_t)(row >> 2));
        }
      }
    }
  }
}

// Single-pass form for the common shapes: every plane fits one pass of V
// chunks per lane (bf16 rows up to 14 KB: V0 = 14; fp8: 7 KB codes with
// V0 = 7 and 224 B scales with V1 = 1). No loop over planes or passes.
// This exact shape (raw pointer arguments, both rows loaded, then a loop
// over the two tokens selecting the register set) measured 99-100 us at
// decode scale against 103-106 us for the general kernel and for variants
// that preload the send positions or unroll the stores.
template <int V>
__device__ __forceinline__ void pack_pass(const uint8_t* x, uint8_t* send, const int32_t* sp,
                                          int tok0, bool two, int T, int R, int row) {
  const int TR = T * R;
  const int n16 = row >> 4;
  RowRegs<V> r0, r1;
  load_row16<V, kPackNtLoads>(r0, (const u32x4*)(x + (size_t)tok0 * row), 0, n16);
  if (two) load_row16<V, kPackNtLoads>(r1, (const u32x4*)(x + (size_t)(tok0 + 1) * row), 0, n16);
  for (int u = 0; u < (two ? 2 : 1); ++u) {
    const int tok = tok0 + u;
    const int s = tok / T;
    for (int k = 0; k < R; ++k) {
      const int p = sp[(size_t)tok * R + k];
      if (p < 0 || p >= TR) continue;
      store_row16(u ? r1 : r0, (u32x4*)(send + ((size_t)s * TR + p) * row), 0, n16);
    }
  }
}

template <int V0>
__global__ __launch_bounds__(kBlock) void pack_fast1_kernel(const uint8_t* x, uint8_t* send,
                                                            const int32_t* sp, int NT, int T,
                                                            int R, int row) {
  const int tok0 = 2 * wave_index();
  if (tok0 >= NT) return;
  pack_pass<V0>(x, send, sp, tok0, tok0 + 1 < NT, T, R, row);
}

template <int V0, int V1>
__global__ __launch_bounds__(kBlock) void pack_fast2_kernel(const uint8_t* x0, uint8_t* send0,
                                                            const uint8_t* x1, uint8_t* send1,
                                                            const int32_t* sp, int NT, int T,
                                                            int R, int row0, int row1) {
  const int tok0 = 2 * wave_index();
  if (tok0 >= NT) return;
  pack_pass<V0>(x0, send0, sp, tok0, tok0 + 1 < NT, T, R, row0);
  pack_pass<V1>(x1, send1, sp, tok0, tok0 + 1 < NT, T, R, row1);
}

// Dispatch in one go for sources whose slots fit one plan chunk: after the
// send side of the plan (own counts, offsets and positions), the first N
// blocks of this kernel do the count exchange and write the receive side of
// the plan (the receiver needs it, the sender does not) while the other
// blocks move the rows, one wave per token pair as in pack_fast1/2. The
// exchange (a latency-bound ~10 us) so hides under the bandwidth-bound
// sender instead of delaying it. V1 = 0: one payload plane.
template <int V0, int V1>
__global__ __launch_bounds__(kBlock) void pack_exchange_kernel(
    const uint8_t* x0, uint8_t* send0, const uint8_t* x1, uint8_t* send1, PlanPtrs p, int N,
    int E, int L, int T, int R, int64_t cap, int row0, int row1, int32_t* status) {
  extern __shared__ int32_t lds[];
  const int b = blockIdx.x;
  if (b < N) {  // block-uniform
    exchange_block<kBlock>(b, 0, b, N, N, E, L, (int64_t)T * R, cap, p, status, lds);
    return;
  }
  const int tok0 = 2 * wave_uniform((b - N) * kWavesPerBlock + (int)threadIdx.x / kWave);
  const int NT = N * T;
  if (tok0 >= NT) return;
  pack_pass<V0>(x0, send0, p.send_pos, tok0, tok0 + 1 < NT, T, R, row0);
  if (V1 > 0) pack_pass<(V1 > 0 ? V1 : 1)>(x1, send1, p.send_pos, tok0, tok0 + 1 < NT, T, R, row1);
}

// XCD-aware block order. A launch's workgroups go to gfx950's 8 XCDs in
// turn (block b runs on XCD b mod 8), and each XCD has its own L2.
// Renumbering block b as (b mod 8) * nb/8 + b/8 hands XCD x the x-th eighth
// of the work, in order. nb must be a multiple of 8.
__device__ __forceinline__ int xcd_block(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

// Division of n < 2^31 by a divisor d >= 1 fixed at launch, with one
// multiply-high, an add and a shift (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994: with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l).
struct FastDiv {
  uint32_t m, l;
};

FastDiv fast_div_of(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  return FastDiv{(uint32_t)((((1ull << l) - d) << 32) / d + 1), l};
}

__device__ __forceinline__ int fast_div(int n, FastDiv f) {
  return (int)(((uint64_t)__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.l);
}

// Sender in send order. The send buffers of all sources are one array of
// N T R rows; wave w writes the w-th 1 KB piece of a plane's rows (one
// 16-byte chunk per lane), reading the token row that send_slot names.
// Measured on gfx950 (decode scale, 32 x 1024 send rows of 14 KB):
//   - stores that advance through memory as one front (consecutive waves on
//     consecutive pieces) run faster than whole rows per wave: a fill writes
//     6.8 TB/s with 1 KB per wave against 5.3 TB/s with 14 KB;
//   - each token row is read R times, from L2 (ordinary cached loads), and
//     the XCD renumbering makes each XCD work through whole sources, so the
//     rows it re-reads stay in its own L2;
//   - the sender so takes 73 us against 99 us for the token-order sender
//     (one wave per token pair, R stores per row); 2 KB and 7 KB pieces per
//     wave took 76 and 78 us.
// Those figures are for back-to-back steps, where each XCD's L2 still holds
// token rows of the previous step (the receiver and the combine access
// memory non-temporally and leave them). After a pass that evicts the
// caches the token rows' first reads come from HBM: 119 us against 104 us
// for the token-order sender, while whole steps (dispatch and combine) stay
// ahead, 346 against 352 us. Extra waves that pre-read each source's rows
// before its range recovered 14 us of that step but cost 6 us back to back.
// The fp8 scale plane (rows of H/32 bytes) is too narrow for pieces: there
// each lane moves one unit (16 bytes, or 4 when the row is not a multiple of
// 16) of the plane's rows in address order, so every wave writes whole lines.
struct MovePlane {
  const uint8_t* src;
  uint8_t* dst;
  FastDiv per_row_div;
  int unit;     // bytes per lane access in the unit path: 16 or 4
  int per_row;  // pieces per row (piece path) or units per row (unit path)
  int n16;      // 16-byte chunks per row (piece path)
  int pieces;   // 1: piece path; 0: unit path
  int waves;    // waves covering the plane
  int blocks;   // blocks covering it, a multiple of 8
};

// Private regions of a split dispatch: send row p of s that is row i < P of
// the segment s -> d (send_seg[s][p] = d T R + i) lives in d's region for s,
// priv[q][((d N + s) P + i) row], instead of the send buffer.
struct PrivRegions {
  uint8_t* priv[2];
  const int32_t* send_seg;
  FastDiv tr_div;
  int TR, N, P;
};

// Row `g` (s T R + p) of plane q: in the private region when it is among the
// first P rows of its segment, else `fallback` (its send-buffer row). An out
// of range send_seg entry keeps the fallback.
__device__ __forceinline__ uint8_t* split_dst(const PrivRegions& v, int q, int g, size_t row,
                                              uint8_t* fallback) {
  const int seg = v.send_seg[g];
  const int d = fast_div(seg, v.tr_div);
  const int i = seg - d * v.TR;
  if (seg < 0 || d >= v.N || i >= v.P) return fallback;
  const int s = fast_div(g, v.tr_div);
  return v.priv[q] + (((size_t)d * v.N + s) * v.P + i) * row;
}

struct GatherArgs {
  MovePlane pl[2];
  const int32_t* send_slot;
  const int2* win_list;  // windowed order for plane 0 (pieces), or null
  FastDiv r_div;
  int NT, NTR;
  PrivRegions split;
};

template <bool SPLIT>
__device__ __forceinline__ void gather_wave(const GatherArgs& a, const MovePlane& pl, int q,
                                            int w) {
  if (pl.pieces) {
    const int j = wave_uniform(fast_div(w, pl.per_row_div));  // send row or list entry
    const int base = (w - j * pl.per_row) * kWave;
    int g, tok;
    if (a.win_list != nullptr && q == 0) {
      const int2 e = a.win_list[j];
      g = wave_uniform(e.x);
      tok = wave_uniform(e.y);
      if (g < 0 || g >= a.NTR || tok < 0 || tok >= a.NT) return;
    } else {
      g = j;
      const int slot = wave_uniform(a.send_slot[g]);
      if (slot < 0) return;  // a row its source does not fill
      tok = fast_div(slot, a.r_div);
      if (tok >= a.NT) return;
    }
    const size_t row = (size_t)pl.n16 * 16;
    uint8_t* dst = pl.dst + (size_t)g * row;
    if (SPLIT) dst = split_dst(a.split, q, g, row, dst);
    RowRegs<1> r;
    load_row16<1, false>(r, (const u32x4*)(pl.src + (size_t)tok * row), base, pl.n16);
    store_row16(r, (u32x4*)dst, base, pl.n16);
    return;
  }
  const int64_t c = (int64_t)w * kWave + lane_id();
  if (c >= (int64_t)a.NTR * pl.per_row) return;
  const int g = (int)(c / pl.per_row);
  const int u = (int)(c - (int64_t)g * pl.per_row);
  const int slot = a.send_slot[g];
  if (slot < 0) return;
  const int tok = fast_div(slot, a.r_div);
  if (tok >= a.NT) return;
  const size_t src = (size_t)tok * pl.per_row + u;
  uint8_t* dst = pl.dst + (size_t)g * pl.per_row * pl.unit;
  if (SPLIT) dst = split_dst(a.split, q, g, (size_t)pl.per_row * pl.unit, dst);
  if (pl.unit == 16)
    store_stream((u32x4*)dst + u, ((const u32x4*)pl.src)[src]);
  else
    __builtin_nontemporal_store(((const uint32_t*)pl.src)[src], (uint32_t*)dst + u);
}

// Blocks [0, xblocks) do the count exchange when EXCHANGE (blocks < N; the
// rest of them idle, so xblocks, a multiple of 8, keeps the XCD of every
// later block equal to its index mod 8); then the blocks of plane 0, then of
// plane 1, each range renumbered per XCD.
// At most 64 VGPRs (8 waves per SIMD): the exchange code would otherwise
// set the register count, and so the occupancy, of every sender wave.
template <bool EXCHANGE, bool SPLIT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(8))) void
pack_gather_kernel(GatherArgs a, PlanPtrs p, int N, int E, int L, int T, int R, int64_t cap,
                   int xblocks, int32_t* status) {
  extern __shared__ int32_t lds[];
  int b = blockIdx.x;
  if (EXCHANGE) {
    if (b < xblocks) {  // block-uniform
      if (b < N) exchange_block<kBlock>(b, 0, b, N, N, E, L, (int64_t)T * R, cap, p, status, lds);
      return;
    }
    b -= xblocks;
  }
  if (b < a.pl[0].blocks) {
    const int w = xcd_block(b, a.pl[0].blocks) * kWavesPerBlock + (int)threadIdx.x / kWave;
    if (w < a.pl[0].waves) gather_wave<SPLIT>(a, a.pl[0], 0, w);
  } else {
    b -= a.pl[0].blocks;
    if (b >= a.pl[1].blocks) return;
    const int w = xcd_block(b, a.pl[1].blocks) * kWavesPerBlock + (int)threadIdx.x / kWave;
    if (w < a.pl[1].waves) gather_wave<SPLIT>(a, a.pl[1], 1, w);
  }
}

// Receiver in receive order with 1 KB pieces: wave w moves the w-th 1 KB
// piece of the delivered rows (recv_rows[j]: send row, grouped row of the
// j-th delivered row), so the grouped buffers fill front to back while the
// pulls from the send buffers are the scattered side. One 8-byte table load
// per wave names both rows. The fp8 scale plane takes the unit path (each
// lane one 16- or 4-byte unit, rows in receive order). Reads are
// non-temporal: every send row is read once. Every row index is range
// checked. Measured at decode scale: 152.8 us against 158.0 us for 7 KB row
// segments per wave (two levels of table loads: grp_slot, then send_pos and
// comb_row); with fp8 rows 80.3 against 85.8 us.
struct RecvArgs {
  MovePlane pl[2];
  const int2* recv_rows;
  int NTR;
  int64_t rows_out;
  PrivRegions split;  // SPLIT: rows a sender left in the private regions
};

template <bool SPLIT>
__device__ __forceinline__ void recv_wave(const RecvArgs& a, const MovePlane& pl, int q, int w) {
  if (pl.pieces) {
    const int j = wave_uniform(fast_div(w, pl.per_row_div));
    const int base = (w - j * pl.per_row) * kWave;
    const int2 r = a.recv_rows[j];
    const int src = wave_uniform(r.x), dst = wave_uniform(r.y);
    if (src < 0 || src >= a.NTR || dst < 0 || dst >= a.rows_out) return;
    const size_t row = (size_t)pl.n16 * 16;
    const uint8_t* from = pl.src + (size_t)src * row;
    if (SPLIT) from = split_dst(a.split, q, src, row, (uint8_t*)from);
    RowRegs<1> v;
    load_row16<1, true>(v, (const u32x4*)from, base, pl.n16);
    store_row16(v, (u32x4*)(pl.dst + (size_t)dst * row), base, pl.n16);
    return;
  }
  const int64_t c = (int64_t)w * kWave + lane_id();
  if (c >= (int64_t)a.NTR * pl.per_row) return;
  const int j = (int)(c / pl.per_row);
  const int u = (int)(c - (int64_t)j * pl.per_row);
  const int2 r = a.recv_rows[j];
  if (r.x < 0 || r.x >= a.NTR || r.y < 0 || r.y >= a.rows_out) return;
  const size_t row = (size_t)pl.per_row * pl.unit;
  const uint8_t* from = pl.src + (size_t)r.x * row;
  if (SPLIT) from = split_dst(a.split, q, r.x, row, (uint8_t*)from);
  uint8_t* to = pl.dst + (size_t)r.y * row;
  if (pl.unit == 16)
    store_stream((u32x4*)to + u, load_stream((const u32x4*)from + u));
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load((const uint32_t*)from + u),
                                (uint32_t*)to + u);
}

// Blocks of plane 0, then of plane 1.
template <bool SPLIT>
__global__ __launch_bounds__(kRecvBlock) void recv_rows_kernel(RecvArgs a) {
  int b = blockIdx.x;
  const int q = b < a.pl[0].blocks ? 0 : 1;
  if (q) b -= a.pl[0].blocks;
  const int w = b * kRecvWaves + (int)threadIdx.x / kWave;
  if (w < a.pl[q].waves) recv_wave<SPLIT>(a, a.pl[q], q, w);
}

// The staged receive path, with the same 1 KB pieces. Send row g = s T R + p
// is row i of the segment s -> d (send_seg[g] = d T R + i) and sits at row
// recv_off[d][s] + i of d's receive buffer; rows at or beyond cap are not
// there (dropped). One send_seg load per wave names the rank and the index.
struct StagedArgs {
  MovePlane pl[2];
  const int32_t* send_seg;
  const int32_t* recv_off;
  const int2* recv_rows;
  FastDiv tr_div;
  int TR, N, NTR;
  int64_t cap;
};

// Receive-buffer row (d cap + r) of send row g, or -1.
__device__ __forceinline__ int64_t staged_row(const StagedArgs& a, int g) {
  const int seg = a.send_seg[g];
  if (seg < 0) return -1;
  const int d = fast_div(seg, a.tr_div);
  if (d >= a.N) return -1;
  const int i = seg - d * a.TR;
  const int s = fast_div(g, a.tr_div);
  const int64_t r = (int64_t)a.recv_off[(size_t)d * (a.N + 1) + s] + i;
  return r >= 0 && r < a.cap ? (int64_t)d * a.cap + r : -1;
}

// TRANSFER: the network write, in send order (wave w: piece of send row
// w / per_row). Otherwise the receiver shuffle, in receive order
// (recv_rows); a delivered grouped row whose receive-buffer row was dropped
// (at or beyond cap) is written as zeros, so it holds no stale bytes.
template <bool TRANSFER>
__device__ __forceinline__ void staged_wave(const StagedArgs& a, const MovePlane& pl, int w) {
  if (pl.pieces) {
    const int j = wave_uniform(fast_div(w, pl.per_row_div));
    const int base = (w - j * pl.per_row) * kWave;
    int64_t from, to;
    if (TRANSFER) {
      from = j;
      to = staged_row(a, j);
    } else {
      const int2 r = a.recv_rows[j];
      const int g = wave_uniform(r.x);
      if (g < 0 || g >= a.NTR || r.y < 0 || r.y >= (int64_t)a.N * a.cap) return;
      from = staged_row(a, g);
      to = wave_uniform(r.y);
    }
    if (to < 0 || (TRANSFER && from < 0)) return;
    const size_t row = (size_t)pl.n16 * 16;
    RowRegs<1> v;
    if (from >= 0)
      load_row16<1, true>(v, (const u32x4*)(pl.src + (size_t)from * row), base, pl.n16);
    else
      v.v[0] = u32x4{0u, 0u, 0u, 0u};
    store_row16(v, (u32x4*)(pl.dst + (size_t)to * row), base, pl.n16);
    return;
  }
  const int64_t c = (int64_t)w * kWave + lane_id();
  if (c >= (int64_t)a.NTR * pl.per_row) return;
  const int j = (int)(c / pl.per_row);
  const int u = (int)(c - (int64_t)j * pl.per_row);
  int64_t from, to;
  if (TRANSFER) {
    from = j;
    to = staged_row(a, j);
  } else {
    const int2 r = a.recv_rows[j];
    if (r.x < 0 || r.x >= a.NTR || r.y < 0 || r.y >= (int64_t)a.N * a.cap) return;
    from = staged_row(a, r.x);
    to = r.y;
  }
  if (to < 0 || (TRANSFER && from < 0)) return;
  const size_t t = (size_t)to * pl.per_row + u;
  if (from < 0) {
    if (pl.unit == 16)
      store_stream((u32x4*)pl.dst + t, u32x4{0u, 0u, 0u, 0u});
    else
      __builtin_nontemporal_store(0u, (uint32_t*)pl.dst + t);
    return;
  }
  const size_t f = (size_t)from * pl.per_row + u;
  if (pl.unit == 16)
    store_stream((u32x4*)pl.dst + t, load_stream((const u32x4*)pl.src + f));
  else
    __builtin_nontemporal_store(__builtin_nontemporal_load((const uint32_t*)pl.src + f),
                                (uint32_t*)pl.dst + t);
}

template <bool TRANSFER>
__global__ __launch_bounds__(kRecvBlock) void staged_kernel(StagedArgs a) {
  int b = blockIdx.x;
  const int q = b < a.pl[0].blocks ? 0 : 1;
  if (q) b -= a.pl[0].blocks;
  const int w = b * kRecvWaves + (int)threadIdx.x / kWave;
  if (w < a.pl[q].waves) staged_wave<TRANSFER>(a, a.pl[q], w);
}

// Chunks per lane for a single pass over a plane of `row` bytes: 14, 7 or 1;
// 0 if the plane needs the general kernel.
int pass_v(int64_t row) {
  if ((row & 15) != 0) return 0;
  const int64_t n16 = row >> 4;
  if (n16 <= kWave) return 1;
  if (n16 <= kSeg) return kSegV;
  if (n16 <= 2 * kSeg) return 2 * kSegV;
  return 0;
}

// Split dispatch. Rows of the segment s -> d (the rows source s sends to the
// experts of rank d) with index i < P inside the segment live in d's
// private region for s, priv[(d * N + s) * P + i]; the others in the send
// buffer. Source s's segment for d starts at send_off[s][d L].
struct Split {
  uint8_t* priv[2];
  const int32_t* send_off;
  int N, E, L, P;
};

__device__ __forceinline__ uint8_t* split_row(const Split& sp, int q, uint8_t* send, int s, int d,
                                              int p, int TR, size_t row) {
  const int i = p - sp.send_off[(size_t)s * (sp.E + 1) + d * sp.L];
  if (i >= 0 && i < sp.P) return sp.priv[q] + (((size_t)d * sp.N + s) * sp.P + i) * row;
  return send + ((size_t)s * TR + p) * row;
}

// Sender half of a split dispatch: as pack_kernel, with each slot's row
// sent to the private region of its destination when it is among the
// first P rows of its segment.
template <int V>
__device__ __forceinline__ void pack_split_plane(const uint8_t* x, uint8_t* send, const Split& sp,
                                                 int q, const int32_t* __restrict__ idx,
                                                 const int32_t* __restrict__ send_pos, int tok0,
                                                 bool two, int T, int R, size_t row) {
  const int TR = T * R;
  const int n16 = (int)(row >> 4);
  for (int base = 0; base < n16; base += kWave * V) {
    RowRegs<V> r0, r1;
    load_row16<V, kPackNtLoads>(r0, (const u32x4*)(x + (size_t)tok0 * row), base, n16);
    if (two) load_row16<V, kPackNtLoads>(r1, (const u32x4*)(x + (size_t)(tok0 + 1) * row), base, n16);
    for (int u = 0; u < (two ? 2 : 1); ++u) {
      const int tok = tok0 + u;
      const int s = tok / T;
      for (int k = 0; k < R; ++k) {
        const int p = send_pos[(size_t)tok * R + k];
        const int e = idx[(size_t)tok * R + k];
        if (p < 0 || p >= TR || e < 0 || e >= sp.E) continue;
        store_row16(u ? r1 : r0, (u32x4*)split_row(sp, q, send, s, e / sp.L, p, TR, row), base,
                    n16);
      }
    }
  }
}

__global__ __launch_bounds__(kBlock) void pack_split_kernel(Planes pl, Split sp,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ send_pos,
                                                            int NT, int T, int R) {
  const int tok0 = 2 * wave_index();
  if (tok0 >= NT) return;
  const bool two = tok0 + 1 < NT;
  const int TR = T * R;
  for (int q = 0; q < pl.planes; ++q) {
    const size_t row = (size_t)pl.row[q];
    if ((row & 15) == 0) {
      const int n16 = (int)(row >> 4);
      if (n16 > kSeg)
        pack_split_plane<2 * kSegV>(pl.src[q], pl.dst[q], sp, q, idx, send_pos, tok0, two, T, R,
                                    row);
      else if (n16 > kWave)
        pack_split_plane<kSegV>(pl.src[q], pl.dst[q], sp, q, idx, send_pos, tok0, two, T, R, row);
      else
        pack_split_plane<1>(pl.src[q], pl.dst[q], sp, q, idx, send_pos, tok0, two, T, R, row);
    } else {
      for (int u = 0; u < (two ? 2 : 1); ++u) {
        const int tok = tok0 + u;
        for (int k = 0; k < R; ++k) {
          const int p = send_pos[(size_t)tok * R + k];
          const int e = idx[(size_t)tok * R + k];
          if (p < 0 || p >= TR || e < 0 || e >= sp.E) continue;
          copy_row4((const uint32_t*)(pl.src[q] + (size_t)tok * row),
                    (uint32_t*)split_row(sp, q, pl.dst[q], tok / T, e / sp.L, p, TR, row),
                    (int64_t)(row >> 2));
        }
      }
    }
  }
}


// Plain copy with the same per-wave loop as the row copies (7 KB per wave).
__global__ __launch_bounds__(kBlock) void probe_copy_kernel(const u32x4* src, u32x4* dst,
                                                            int64_t n16) {
  const int64_t base = (int64_t)wave_index() * kSeg;
  if (base >= n16) return;
  const int64_t left = n16 - base;
  const int n = left < kSeg ? (int)left : kSeg;
  RowRegs<kSegV> r;
  load_row16(r, src + base, 0, n);
  store_row16(r, dst + base, 0, n);
}

Planes make_planes(const Dims& d, const void* const src[2], void* const dst[2]) {
  Planes p{};
  p.planes = d.planes;
  for (int q = 0; q < 2; ++q) {
    p.src[q] = q < d.planes ? (const uint8_t*)src[q] : nullptr;
    p.dst[q] = q < d.planes ? (uint8_t*)dst[q] : nullptr;
    p.row[q] = q < d.planes ? d.row[q] : 0;
  }
  return p;
}

unsigned blocks_for(int64_t waves) {
  return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}


}  // namespace

hipError_t launch_pack_gather(const Dims& d, const void* const x[2], const PlanPtrs& p,
                              void* const send[2], bool exchange, int32_t* status,
                              hipStream_t stream, const PrivRegions* split = nullptr,
                              bool windowed = false);
bool gather_fits(const Dims& d);

hipError_t launch_pack(const Dims& d, const void* const x[2], const PlanPtrs& p,
                       void* const send[2], hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  if (gather_fits(d)) return launch_pack_gather(d, x, p, send, false, nullptr, stream);
  if (d.win > 0)
    return launch_pack_gather(d, x, p, send, false, nullptr, stream, nullptr, true);
  const dim3 grid(blocks_for((d.NT + 1) / 2));
  const Planes pl = make_planes(d, x, send);
  const int v0 = pass_v(d.row[0]);
  const int v1 = d.planes > 1 ? pass_v(d.row[1]) : -1;
  const uint8_t* x0 = (const uint8_t*)x[0];
  uint8_t* s0 = (uint8_t*)send[0];
  const int NT = (int)d.NT, r0 = (int)d.row[0];
  if (v0 == 2 * kSegV && v1 == -1) {
    hipLaunchKernelGGL(pack_fast1_kernel<2 * kSegV>, grid, dim3(kBlock), 0, stream, x0, s0,
                       p.send_pos, NT, d.T, d.R, r0);
  } else if (v0 == kSegV && v1 == -1) {
    hipLaunchKernelGGL(pack_fast1_kernel<kSegV>, grid, dim3(kBlock), 0, stream, x0, s0,
                       p.send_pos, NT, d.T, d.R, r0);
  } else if (v0 == kSegV && v1 == 1) {
    hipLaunchKernelGGL((pack_fast2_kernel<kSegV, 1>), grid, dim3(kBlock), 0, stream, x0, s0,
                       (const uint8_t*)x[1], (uint8_t*)send[1], p.send_pos, NT, d.T, d.R, r0,
                       (int)d.row[1]);
  } else {
    hipLaunchKernelGGL(pack_kernel, grid, dim3(kBlock), 0, stream, pl, p.send_pos, NT, d.T, d.R);
  }
  return hipGetLastError();
}

// The count exchange can share the sender's launch when every source's
// slots fit one plan chunk and the exchange's LDS stays small (E <= 512).
bool dispatch_fused_fits(const Dims& d) {
  return d.nchunks == 1 && d.TR <= kPlanChunk && d.E <= 512 && d.N <= 1024;
}

// ... and the plain sender has its single-pass form for these rows.
bool pack_exchange_fits(const Dims& d) {
  const int v0 = pass_v(d.row[0]);
  const int v1 = d.planes > 1 ? pass_v(d.row[1]) : 0;
  return dispatch_fused_fits(d) && v0 > 0 && (d.planes == 1 || v1 == 1);
}

// LDS of the exchange with tpb threads per block (see exchange_block).
size_t lds_exchange_bytes(const Dims& d, int tpb) {
  const int groups = d.E >= tpb ? 1 : tpb / d.E;
  return sizeof(int32_t) * ((size_t)4 * (d.E + 1) + (d.N + 1) + tpb / kWave +
                            (size_t)2 * groups * d.E);
}

template <int V0, int V1>
hipError_t launch_pack_exchange_v(const Dims& d, const void* const x[2], const PlanPtrs& p,
                                  void* const send[2], int32_t* status, hipStream_t stream) {
  const unsigned grid = (unsigned)d.N + blocks_for((d.NT + 1) / 2);
  hipLaunchKernelGGL((pack_exchange_kernel<V0, V1>), dim3(grid), dim3(kBlock),
                     lds_exchange_bytes(d, kBlock), stream, (const uint8_t*)x[0], (uint8_t*)send[0],
                     d.planes > 1 ? (const uint8_t*)x[1] : nullptr,
                     d.planes > 1 ? (uint8_t*)send[1] : nullptr, p, d.N, d.E, d.L, d.T, d.R,
                     d.cap, (int)d.row[0], d.planes > 1 ? (int)d.row[1] : 0, status);
  return hipGetLastError();
}

// The send-order sender re-reads each token row R times and relies on an
// XCD's 4 MB L2 holding the rows of the source it works on: used when one
// source's token rows (all planes) take at most kGatherSourceBytes. Measured
// at H = 7168 (bf16) against the token-order sender, whole dispatch +
// combine steps: 1.8 MB per source 90 vs 96 us (8 ranks) and 329 vs 352 us
// (32 ranks); 3.7 MB 170 vs 182 us; 7.3 MB even; 14.7 MB 743 vs 698 us.
// Larger sources take the windowed send order (d.win > 0: the rows of W
// tokens at a time, W of them fitting kGatherSourceBytes) up to
// kWindowSourceBytes per source and kWindowSendBytes of send buffers:
// sender alone, 8 ranks x 1024 tokens 148-153 us against 186 us in token
// order; 32 x 512 tokens 293-298 against 359 us; 8 x 2048 tokens 298
// against 360 us. With send buffers past ~2 GB (8 x 3072 tokens, 2.8 GB)
// the token-order sender measured faster (637 against 707 us).
bool gather_fits(const Dims& d) {
  int64_t bytes = 0;
  for (int q = 0; q < d.planes; ++q) bytes += d.row[q];
  return (int64_t)d.T * bytes <= kGatherSourceBytes;
}

// A plane takes the piece path when its rows hold at least one 1 KB piece
// and are a multiple of 16 bytes; otherwise the unit path. `per_block`:
// waves per workgroup of the kernel that moves it.
MovePlane move_plane(const void* src, void* dst, int64_t row, int64_t NTR,
                     int per_block = kWavesPerBlock) {
  MovePlane g{};
  g.src = (const uint8_t*)src;
  g.dst = (uint8_t*)dst;
  int64_t waves;
  if ((row & 15) == 0 && row >= 16 * kWave) {
    g.pieces = 1;
    g.unit = 16;
    g.n16 = (int)(row >> 4);
    g.per_row = (g.n16 + kWave - 1) / kWave;
    waves = NTR * g.per_row;
  } else {
    g.pieces = 0;
    g.unit = (row & 15) == 0 ? 16 : 4;
    g.per_row = (int)(row / g.unit);
    waves = (NTR * g.per_row + kWave - 1) / kWave;
  }
  g.per_row_div = fast_div_of((uint32_t)g.per_row);
  g.waves = (int)waves;
  g.blocks = (int)(((waves + per_block - 1) / per_block + 7) / 8 * 8);
  return g;
}

hipError_t launch_pack_gather(const Dims& d, const void* const x[2], const PlanPtrs& p,
                              void* const send[2], bool exchange, int32_t* status,
                              hipStream_t stream, const PrivRegions* split, bool windowed) {
  GatherArgs a{};
  if (split != nullptr) a.split = *split;
  for (int q = 0; q < d.planes; ++q) a.pl[q] = move_plane(x[q], send[q], d.row[q], d.NTR);
  // Windowed order: plane 0's pieces walk the work list (one entry per slot
  // of each window, padded); a plane too narrow for pieces keeps send order.
  if (windowed && a.pl[0].pieces && p.win_list != nullptr) {
    a.pl[0] = move_plane(x[0], send[0], d.row[0], (int64_t)d.N * d.nwin * d.win * d.R);
    a.win_list = (const int2*)p.win_list;
  }
  a.send_slot = p.send_slot;
  a.r_div = fast_div_of((uint32_t)d.R);
  a.NT = (int)d.NT;
  a.NTR = (int)d.NTR;
  const int xblocks = exchange ? (d.N + 7) / 8 * 8 : 0;
  const unsigned grid = (unsigned)(xblocks + a.pl[0].blocks + a.pl[1].blocks);
  const size_t lds = exchange ? lds_exchange_bytes(d, kBlock) : 0;
  if (exchange && split == nullptr)
    hipLaunchKernelGGL((pack_gather_kernel<true, false>), dim3(grid), dim3(kBlock), lds, stream, a,
                       p, d.N, d.E, d.L, d.T, d.R, d.cap, xblocks, status);
  else if (split == nullptr)
    hipLaunchKernelGGL((pack_gather_kernel<false, false>), dim3(grid), dim3(kBlock), 0, stream, a,
                       p, d.N, d.E, d.L, d.T, d.R, d.cap, 0, status);
  else
    hipLaunchKernelGGL((pack_gather_kernel<false, true>), dim3(grid), dim3(kBlock), 0, stream, a,
                       p, d.N, d.E, d.L, d.T, d.R, d.cap, 0, status);
  return hipGetLastError();
}

hipError_t launch_recv_rows(const Dims& d, const void* const send[2], const PlanPtrs& p,
                            void* const grouped[2], const PrivRegions* split,
                            hipStream_t stream) {
  if (d.NTR == 0) return hipSuccess;
  RecvArgs a{};
  for (int q = 0; q < d.planes; ++q)
    a.pl[q] = move_plane(send[q], grouped[q], d.row[q], d.NTR, kRecvWaves);
  a.recv_rows = (const int2*)p.recv_rows;
  a.NTR = (int)d.NTR;
  a.rows_out = (int64_t)d.N * d.cap;
  const dim3 grid((unsigned)(a.pl[0].blocks + a.pl[1].blocks));
  if (split == nullptr) {
    hipLaunchKernelGGL(recv_rows_kernel<false>, grid, dim3(kRecvBlock), 0, stream, a);
  } else {
    a.split = *split;
    hipLaunchKernelGGL(recv_rows_kernel<true>, grid, dim3(kRecvBlock), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_recv(const Dims& d, const void* const send[2], const PlanPtrs& p,
                       void* const grouped[2], hipStream_t stream) {
  return launch_recv_rows(d, send, p, grouped, nullptr, stream);
}

hipError_t launch_dispatch(const Dims& d, const int32_t* idx, const void* const x[2],
                           const PlanPtrs& p, void* const send[2], void* const grouped[2],
                           int32_t* status, hipStream_t stream) {
  const bool gather = gather_fits(d) || d.win > 0;
  if (!(pack_exchange_fits(d) || (dispatch_fused_fits(d) && gather)) || d.NT == 0) {
    hipError_t e = launch_plan(d, idx, p, status, stream);
    if (e == hipSuccess) e = launch_pack(d, x, p, send, stream);
    if (e == hipSuccess) e = launch_recv(d, send, p, grouped, stream);
    return e;
  }
  // The send-order sender re-reads each token row R times, and after other
  // work has evicted the memory-side cache (MALL) its first reads of every
  // row wait on HBM. The send-side plan launch is latency-bound and leaves
  // the memory system idle, so it also touches the token rows into the MALL
  // (see launch_plan_local). Measured on the decode workload after a pass
  // that evicts the caches: the sender takes 101.7 us with the rows in HBM
  // and 74.8 us with them in the MALL; whole steps 353.5 against 330 us
  // (back to back, where the rows are in the MALL already, 319.4 against
  // 323.5 us; the all-to-one workload 669 against 643 us, back to back 625
  // against 637 us).
  RowTouch touch{};
  int64_t touch_bytes = 0;
  for (int q = 0; q < d.planes; ++q) {
    touch.src[q] = (const uint8_t*)x[q];
    touch.bytes[q] = (int64_t)d.T * d.row[q];
    touch_bytes += d.N * touch.bytes[q];
  }
  const bool do_touch = gather_fits(d) && touch_bytes <= kTouchMaxBytes;
  hipError_t e = launch_plan_local(d, idx, p, status, stream, true, do_touch ? &touch : nullptr);
  if (e != hipSuccess) return e;
  if (gather) {
    e = launch_pack_gather(d, x, p, send, true, status, stream, nullptr, d.win > 0);
    if (e != hipSuccess) return e;
    return launch_recv(d, send, p, grouped, stream);
  }
  const int v0 = pass_v(d.row[0]);
  const int v1 = d.planes > 1 ? pass_v(d.row[1]) : 0;
  if (v1 == 0) {
    if (v0 == 2 * kSegV) e = launch_pack_exchange_v<2 * kSegV, 0>(d, x, p, send, status, stream);
    else if (v0 == kSegV) e = launch_pack_exchange_v<kSegV, 0>(d, x, p, send, status, stream);
    else e = launch_pack_exchange_v<1, 0>(d, x, p, send, status, stream);
  } else {
    if (v0 == 2 * kSegV) e = launch_pack_exchange_v<2 * kSegV, 1>(d, x, p, send, status, stream);
    else if (v0 == kSegV) e = launch_pack_exchange_v<kSegV, 1>(d, x, p, send, status, stream);
    else e = launch_pack_exchange_v<1, 1>(d, x, p, send, status, stream);
  }
  if (e != hipSuccess) return e;
  return launch_recv(d, send, p, grouped, stream);
}

Split make_split(const Dims& d, void* const priv[2], int P, const PlanPtrs& p) {
  Split sp{};
  for (int q = 0; q < 2; ++q) sp.priv[q] = (P > 0 && q < d.planes) ? (uint8_t*)priv[q] : nullptr;
  sp.send_off = p.send_off;
  sp.N = d.N;
  sp.E = d.E;
  sp.L = d.L;
  sp.P = P;
  return sp;
}

PrivRegions make_priv(const Dims& d, void* const priv[2], int P, const PlanPtrs& p) {
  PrivRegions v{};
  for (int q = 0; q < 2; ++q) v.priv[q] = (P > 0 && q < d.planes) ? (uint8_t*)priv[q] : nullptr;
  v.send_seg = p.send_seg;
  v.tr_div = fast_div_of((uint32_t)(d.TR > 0 ? d.TR : 1));
  v.TR = (int)d.TR;
  v.N = d.N;
  v.P = P;
  return v;
}

hipError_t launch_pack_split(const Dims& d, const int32_t* idx, const void* const x[2],
                             const PlanPtrs& p, void* const send[2], void* const priv[2], int P,
                             hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  if (P == 0) return launch_pack(d, x, p, send, stream);  // no private rows: the plain sender
  if (gather_fits(d) || d.win > 0) {
    const PrivRegions v = make_priv(d, priv, P, p);
    return launch_pack_gather(d, x, p, send, false, nullptr, stream, &v, d.win > 0);
  }
  hipLaunchKernelGGL(pack_split_kernel, dim3(blocks_for((d.NT + 1) / 2)), dim3(kBlock), 0, stream,
                     make_planes(d, x, send), make_split(d, priv, P, p), idx, p.send_pos,
                     (int)d.NT, d.T, d.R);
  return hipGetLastError();
}

hipError_t launch_recv_split(const Dims& d, const void* const send[2], void* const priv[2], int P,
                             const PlanPtrs& p, void* const grouped[2], hipStream_t stream) {
  if (d.NTR == 0) return hipSuccess;
  const PrivRegions v = make_priv(d, priv, P, p);
  return launch_recv_rows(d, send, p, grouped, P > 0 ? &v : nullptr, stream);
}

template <bool TRANSFER>
hipError_t launch_staged(const Dims& d, const void* const src[2], const PlanPtrs& p,
                         void* const dst[2], hipStream_t stream) {
  if (d.NTR == 0) return hipSuccess;
  StagedArgs a{};
  for (int q = 0; q < d.planes; ++q)
    a.pl[q] = move_plane(src[q], dst[q], d.row[q], d.NTR, kRecvWaves);
  a.send_seg = p.send_seg;
  a.recv_off = p.recv_off;
  a.recv_rows = (const int2*)p.recv_rows;
  a.tr_div = fast_div_of((uint32_t)d.TR);
  a.TR = (int)d.TR;
  a.N = d.N;
  a.NTR = (int)d.NTR;
  a.cap = d.cap;
  hipLaunchKernelGGL(staged_kernel<TRANSFER>, dim3((unsigned)(a.pl[0].blocks + a.pl[1].blocks)),
                     dim3(kRecvBlock), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_transfer(const Dims& d, const void* const send[2], const PlanPtrs& p,
                           void* const recv[2], hipStream_t stream) {
  return launch_staged<true>(d, send, p, recv, stream);
}

hipError_t launch_unpack(const Dims& d, const void* const recv[2], const PlanPtrs& p,
                         void* const grouped[2], hipStream_t stream) {
  return launch_staged<false>(d, recv, p, grouped, stream);
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t waves = (n16 + kSeg - 1) / kSeg;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks_for(waves)), dim3(kBlock), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace ep
