// Dispatch data movement: sender pack, the per-pair transfer, the receiver
// unpack, and the receiver with the transfer fused in (pull).
//
// Method: "Enabling trillion-parameter models on AWS EFA", section
// "Dispatch and combine": the sender shuffles tokens into a send buffer laid
// out so that each peer takes one bulk write; the receiver shuffles its
// receive buffer into the grouped-GEMM input; within a node, buffers mapped
// into the peers let a rank pull tokens directly.
//
// All kernels move whole rows as opaque bytes. One wave owns one row: lane l
// moves 16-byte chunks l, l+64, ..., and every chunk of the row is loaded
// before the first store, so a 14 KB bf16 row (H = 7168) is one round trip.
// Row indices are wave-uniform and live in scalar registers.
#include "ep_device.hpp"
#include "ep_kernels.hpp"

namespace ep {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
constexpr int kRowV = 14;  // 16-byte chunks per lane per pass: 14 KB per wave

struct Planes {
  const uint8_t* src[2];
  uint8_t* dst[2];
  int64_t row[2];
  int planes;
};

__device__ __forceinline__ int wave_index() {
  return wave_uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
}

// Copy one row of n16 16-byte chunks with the whole wave, V chunks per lane
// per pass.
template <int V>
__device__ __forceinline__ void copy_row16(const uint8_t* src, uint8_t* dst, int n16) {
  for (int base = 0; base < n16; base += kWave * V) {
    RowRegs<V> r;
    load_row16(r, (const u32x4*)src, base, n16);
    store_row16(r, (u32x4*)dst, base, n16);
  }
}

// Copy one row of `row` bytes (multiple of 4) with the whole wave. The
// chunks per lane follow the row size (14 for a 14 KB bf16 row, 7 for a
// 7 KB fp8 row, 1 for a scale row), so no wave issues store instructions
// whose lanes would all be clamped duplicates.
__device__ __forceinline__ void wave_copy_row(const uint8_t* src, uint8_t* dst, int64_t row) {
  if ((row & 15) == 0) {
    const int n16 = (int)(row >> 4);
    if (n16 > kWave * 7)
      copy_row16<kRowV>(src, dst, n16);
    else if (n16 > kWave)
      copy_row16<7>(src, dst, n16);
    else
      copy_row16<1>(src, dst, n16);
  } else {
    copy_row4((const uint32_t*)src, (uint32_t*)dst, row >> 2);
  }
}

// Sender: one wave per pair of tokens. Both token rows are loaded (28 KB in
// flight per wave), then each is written to its R send slots. Two tokens
// per wave measured faster than one (more loads in flight per wave at the
// same occupancy). send rows of source s start at s * T * R.
template <int V>
__device__ __forceinline__ void pack_stores(const RowRegs<V>& r, uint8_t* dst0, const int32_t* sp,
                                            int R, int64_t TR, int64_t row, int base, int n16) {
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
                                           bool two, int T, int R, int64_t row) {
  const int64_t TR = (int64_t)T * R;
  const int n16 = (int)(row >> 4);
  for (int base = 0; base < n16; base += kWave * V) {
    RowRegs<V> r0, r1;
    load_row16(r0, (const u32x4*)(x + (size_t)tok0 * row), base, n16);
    if (two) load_row16(r1, (const u32x4*)(x + (size_t)(tok0 + 1) * row), base, n16);
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
  const int64_t TR = (int64_t)T * R;
  for (int q = 0; q < pl.planes; ++q) {
    const int64_t row = pl.row[q];
    if ((row & 15) == 0) {
      const int n16 = (int)(row >> 4);
      if (n16 > kWave * 7)
        pack_plane<kRowV>(pl.src[q], pl.dst[q], send_pos, tok0, two, T, R, row);
      else if (n16 > kWave)
        pack_plane<7>(pl.src[q], pl.dst[q], send_pos, tok0, two, T, R, row);
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
                    (uint32_t*)(dst0 + (size_t)p * row), row >> 2);
        }
      }
    }
  }
}

// Receiver with the transfer fused in: wave j pulls the j-th row of the
// receive order (grp_slot: each rank's grouped rows in turn) from its
// source's send buffer into the grouped layout on its expert's rank
// (comb_row = rank * cap + grouped position). Visiting rows in receive
// order makes every rank's grouped buffer a sequential write stream (the
// pulls from the send buffers are the scattered side, which costs less).
// Every row index is range checked, so no plan content can make the kernel
// leave its buffers.
__global__ __launch_bounds__(kBlock) void recv_kernel(Planes pl, const int32_t* __restrict__ grp_slot,
                                                      const int32_t* __restrict__ send_pos,
                                                      const int32_t* __restrict__ comb_row,
                                                      int NTR, int TR, int64_t rows_out) {
  const int j = wave_index();
  if (j >= NTR) return;
  const int slot = grp_slot[j];
  if (slot < 0 || slot >= NTR) return;
  const int p = send_pos[slot];
  const int g = comb_row[slot];
  if (p < 0 || p >= TR || g < 0 || g >= rows_out) return;
  const int s = slot / TR;
  for (int q = 0; q < pl.planes; ++q) {
    const int64_t row = pl.row[q];
    wave_copy_row(pl.src[q] + ((size_t)s * TR + p) * row, pl.dst[q] + (size_t)g * row, row);
  }
}

// The network write: send row i of source s lies in the segment of the rank
// d with send_off[s][dL] <= i < send_off[s][(d+1)L] and lands in d's receive
// buffer at recv_off[d][s] + (i - send_off[s][dL]).
__global__ __launch_bounds__(kBlock) void transfer_kernel(Planes pl, const int32_t* __restrict__ send_off,
                                                          const int32_t* __restrict__ recv_off,
                                                          int N, int E, int L, int64_t TR,
                                                          int64_t cap) {
  const int g = wave_index();
  if (g >= (int64_t)N * TR) return;
  const int s = (int)(g / TR);
  const int i = (int)(g - (int64_t)s * TR);
  const int32_t* so = send_off + (size_t)s * (E + 1);
  if (i >= so[E]) return;
  int lo = 0, hi = N - 1;  // largest d with so[d * L] <= i
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (so[mid * L] <= i) lo = mid; else hi = mid - 1;
  }
  const int d = lo;
  const int64_t r = (int64_t)recv_off[(size_t)d * (N + 1) + s] + (i - so[d * L]);
  if (r < 0 || r >= cap) return;
  for (int q = 0; q < pl.planes; ++q) {
    const int64_t row = pl.row[q];
    wave_copy_row(pl.src[q] + ((size_t)s * TR + i) * row,
                  pl.dst[q] + ((size_t)d * cap + r) * row, row);
  }
}

// Receiver on a materialised receive buffer. Row r of rank d came from the
// source s with recv_off[d][s] <= r < recv_off[d][s+1]; inside s's segment it
// is send row send_off[s][dL] + (r - recv_off[d][s]), whose expert e gives
// the grouped row grp_off[d][e - dL] + src_off[s][e] + (rank within e).
__global__ __launch_bounds__(kBlock) void unpack_kernel(Planes pl, const int32_t* __restrict__ send_off,
                                                        const int32_t* __restrict__ recv_off,
                                                        const int32_t* __restrict__ grp_off,
                                                        const int32_t* __restrict__ src_off,
                                                        int N, int E, int L, int64_t cap) {
  const int d = blockIdx.y;
  const int r = wave_index();
  const int32_t* ro = recv_off + (size_t)d * (N + 1);
  const int64_t lim = ro[N] < cap ? ro[N] : cap;
  if (r >= lim) return;
  int lo = 0, hi = N - 1;  // largest s with ro[s] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ro[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const int32_t* so = send_off + (size_t)s * (E + 1);
  const int i = so[d * L] + (r - ro[s]);
  int elo = d * L, ehi = d * L + L - 1;  // largest e of rank d with so[e] <= i
  while (elo < ehi) {
    const int mid = (elo + ehi + 1) >> 1;
    if (so[mid] <= i) elo = mid; else ehi = mid - 1;
  }
  const int e = elo;
  const int64_t gpos = (int64_t)grp_off[(size_t)d * (L + 1) + (e - d * L)] +
                       src_off[(size_t)s * E + e] + (i - so[e]);
  if (gpos < 0 || gpos >= cap) return;
  for (int q = 0; q < pl.planes; ++q) {
    const int64_t row = pl.row[q];
    wave_copy_row(pl.src[q] + ((size_t)d * cap + r) * row,
                  pl.dst[q] + ((size_t)d * cap + gpos) * row, row);
  }
}

__global__ __launch_bounds__(kBlock) void probe_copy_kernel(const u32x4* src, u32x4* dst,
                                                            int64_t n16) {
  const int64_t base = (int64_t)wave_index() * kWave * kRowV;
  if (base >= n16) return;
  const int64_t left = n16 - base;
  const int n = left < kWave * kRowV ? (int)left : kWave * kRowV;
  RowRegs<kRowV> r;
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

hipError_t launch_pack(const Dims& d, const void* const x[2], const PlanPtrs& p,
                       void* const send[2], hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_kernel, dim3(blocks_for((d.NT + 1) / 2)), dim3(kBlock), 0, stream,
                     make_planes(d, x, send), p.send_pos, (int)d.NT, d.T, d.R);
  return hipGetLastError();
}

hipError_t launch_recv(const Dims& d, const void* const send[2], const PlanPtrs& p,
                       void* const grouped[2], hipStream_t stream) {
  if (d.NTR == 0) return hipSuccess;
  hipLaunchKernelGGL(recv_kernel, dim3(blocks_for(d.NTR)), dim3(kBlock), 0, stream,
                     make_planes(d, send, grouped), p.grp_slot, p.send_pos, p.comb_row,
                     (int)d.NTR, (int)d.TR, (int64_t)d.N * d.cap);
  return hipGetLastError();
}

hipError_t launch_transfer(const Dims& d, const void* const send[2], const PlanPtrs& p,
                           void* const recv[2], hipStream_t stream) {
  if (d.NTR == 0) return hipSuccess;
  hipLaunchKernelGGL(transfer_kernel, dim3(blocks_for(d.NTR)), dim3(kBlock), 0, stream,
                     make_planes(d, send, recv), p.send_off, p.recv_off, d.N, d.E, d.L, d.TR,
                     d.cap);
  return hipGetLastError();
}

hipError_t launch_unpack(const Dims& d, const void* const recv[2], const PlanPtrs& p,
                         void* const grouped[2], hipStream_t stream) {
  const int64_t rows = d.cap < d.NTR ? d.cap : d.NTR;  // no rank holds more
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks_for(rows), d.N), dim3(kBlock), 0, stream,
                     make_planes(d, recv, grouped), p.send_off, p.recv_off, p.grp_off,
                     p.src_off, d.N, d.E, d.L, d.cap);
  return hipGetLastError();
}

hipError_t launch_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t waves = (n16 + kWave * kRowV - 1) / (kWave * kRowV);
  hipLaunchKernelGGL(probe_copy_kernel, dim3(blocks_for(waves)), dim3(kBlock), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError();
}

}  // namespace ep
