// Combine receiver and the stand-in expert.
//
// Method: "Enabling trillion-parameter models on AWS EFA", section
// "Dispatch and combine": with the routing known from dispatch, combine
// returns each token's expert outputs to its source rank and accumulates
// their routing-weighted average into the output tensor; accumulation
// happens on the receiving (source) side only.
//
// Two waves per output token (seven at prefill scale, see launch_combine),
// each owning alternate column blocks of 64 x V 16-byte chunks (for H = 7168
// and V = 7 each wave takes one half of the row). Per
// block the wave loads two of the token's expert rows at a time (both in
// flight) and accumulates w_k * y_k in fp32 with fused multiply-adds in k
// order, then rounds once to bf16 (nearest, ties to even) and stores 16
// bytes per lane. Splitting a token over two waves doubles the waves in
// flight at 120 VGPRs per wave; keeping more rows in flight per wave
// instead costs occupancy and measured slower.
#include "ep_device.hpp"
#include "ep_kernels.hpp"

namespace ep {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
constexpr int kCombV = 7;          // 16-byte chunks (8 bf16) per lane per block
constexpr int kCombWaves = 2;      // waves per output token
constexpr int kCombRows = 2;       // expert rows in flight per wave
constexpr int kPresumV = 1;        // presum_rows_kernel: chunks per lane per block
constexpr int kPresumW = 14;       // and waves per token

__device__ __forceinline__ int wave_index() {
  return wave_uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
}

template <int V>
__device__ __forceinline__ void fma_row(float (&acc)[V][8], const RowRegs<V>& r, float w) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[i][2 * h] = __builtin_fmaf(w, bf16_lo(r.v[i][h]), acc[i][2 * h]);
      acc[i][2 * h + 1] = __builtin_fmaf(w, bf16_hi(r.v[i][h]), acc[i][2 * h + 1]);
    }
  }
}

template <int V>
__device__ __forceinline__ void store_acc(float (&acc)[V][8], u32x4* o, int base, int n16) {
  RowRegs<V> res;
#pragma unroll
  for (int i = 0; i < V; ++i)
#pragma unroll
    for (int h = 0; h < 4; ++h)
      res.v[i][h] = f32_to_bf16_bits(acc[i][2 * h]) | (f32_to_bf16_bits(acc[i][2 * h + 1]) << 16);
  store_row16(res, o, base, n16);
}

// V chunks per lane per column block, W waves per token, ROWS expert rows
// in flight per wave.
template <int V, int W, int ROWS>
__global__ __launch_bounds__(kBlock) void combine_kernel(const uint16_t* y, const float* w,
                                                         const int32_t* comb_row, uint16_t* out,
                                                         int NT, int R, int H, int64_t rows_in) {
  const int wv = wave_index();
  const int tok = wv / W;
  const int part = wv % W;
  if (tok >= NT) return;
  const int32_t* rows = comb_row + (size_t)tok * R;
  const float* wt = w + (size_t)tok * R;
  const int n16 = H / 8;
  const u32x4* ybase = (const u32x4*)y;
  u32x4* o = (u32x4*)(out + (size_t)tok * H);
  for (int base = part * kWave * V; base < n16; base += W * kWave * V) {
    float acc[V][8];
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int k0 = 0; k0 < R; k0 += ROWS) {
      // Rows k0 .. k0 + ROWS - 1: loads of all in flight, then the FMAs.
      // Rows outside [0, rows_in) (dropped slots) contribute nothing.
      RowRegs<V> v[ROWS];
#pragma unroll
      for (int b = 0; b < ROWS; ++b)
        if (k0 + b < R && rows[k0 + b] >= 0 && rows[k0 + b] < rows_in)
          load_row16(v[b], ybase + (size_t)rows[k0 + b] * n16, base, n16);
#pragma unroll
      for (int b = 0; b < ROWS; ++b)
        if (k0 + b < R && rows[k0 + b] >= 0 && rows[k0 + b] < rows_in)
          fma_row(acc, v[b], wt[k0 + b]);
    }
    store_acc(acc, o, base, n16);
  }
}

// Combine with partial sums on the expert side ("Evaluation": sender-side
// accumulation moves fewer bytes than accumulating on the receiver only).
// A token's slots whose expert rows live on the same rank form a group;
// rows[k] = rank * cap + grouped position, so the rank is rows[k] / cap.
// The group's first slot is its leader.
__device__ __forceinline__ bool slot_ok(int r, int64_t rows_in) { return r >= 0 && r < rows_in; }

__device__ __forceinline__ bool is_leader(const int32_t* rows, int k, int cap, int64_t rows_in) {
  const int rk = rows[k];
  if (!slot_ok(rk, rows_in)) return false;
  const int d = rk / cap;
  for (int k2 = 0; k2 < k; ++k2) {
    const int r2 = rows[k2];
    if (slot_ok(r2, rows_in) && r2 / cap == d) return false;
  }
  return true;
}

// Expert side: for each group, sum w_k * y_k over its slots in k order
// (fused multiply-adds from 0, fp32), round once to bf16 and store the row
// at the leader's slot of `partial` ([N][T R][H]). Two waves per token as
// in combine_kernel; one expert row in flight per lane set.
__global__ __launch_bounds__(kBlock) void presum_kernel(const uint16_t* y, const float* w,
                                                        const int32_t* comb_row,
                                                        uint16_t* partial, int NT, int R, int H,
                                                        int cap, int64_t rows_in) {
  const int wv = wave_index();
  const int tok = wv / kCombWaves;
  const int part = wv % kCombWaves;
  if (tok >= NT) return;
  const int32_t* rows = comb_row + (size_t)tok * R;
  const float* wt = w + (size_t)tok * R;
  const int n16 = H / 8;
  const u32x4* ybase = (const u32x4*)y;
  for (int k0 = 0; k0 < R; ++k0) {
    if (!is_leader(rows, k0, cap, rows_in)) continue;
    const int d = rows[k0] / cap;
    u32x4* o = (u32x4*)(partial + ((size_t)tok * R + k0) * H);
    for (int base = part * kWave * kCombV; base < n16; base += kCombWaves * kWave * kCombV) {
      float acc[kCombV][8];
#pragma unroll
      for (int i = 0; i < kCombV; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
      for (int k = k0; k < R; ++k) {
        const int rk = rows[k];
        if (!slot_ok(rk, rows_in) || rk / cap != d) continue;
        RowRegs<kCombV> v;
        load_row16(v, ybase + (size_t)rk * n16, base, n16);
        fma_row(acc, v, wt[k]);
      }
      store_acc(acc, o, base, n16);
    }
  }
}

// Expert side with every expert row of a token in flight (R <= kPresumMaxR):
// wave part of token tok owns column blocks of 64 x V chunks; per block it
// loads the token's R rows, then for each group (leader k0, in k order) sums
// w_k * y_k over the group's slots in k order with fused multiply-adds from
// 0, rounds once to bf16 and stores the leader's partial row. The same
// arithmetic as presum_kernel, so the same bits. Measured (whole partial-sum
// combine, expert and source side): decode 258-267 us against 271 us with
// presum_kernel, prefill 1609-1621 against 1701 us; 1 chunk per lane and 14
// waves per token against 2 and 7: 258-263 against 264-267 us at decode. The
// same shape for the source side was slower at prefill (1702-1708 us).
constexpr int kPresumMaxR = 8;

template <int V, int W>
__global__ __launch_bounds__(kBlock) void presum_rows_kernel(const uint16_t* y, const float* w,
                                                             const int32_t* comb_row,
                                                             uint16_t* partial, int NT, int R,
                                                             int H, int cap, int64_t rows_in) {
  const int wv = wave_index();
  const int tok = wv / W;
  const int part = wv % W;
  if (tok >= NT) return;
  const int32_t* rows = comb_row + (size_t)tok * R;
  const float* wt = w + (size_t)tok * R;
  int rk[kPresumMaxR], dk[kPresumMaxR];
  float wk[kPresumMaxR];
#pragma unroll
  for (int k = 0; k < kPresumMaxR; ++k) {
    rk[k] = k < R ? rows[k] : -1;
    wk[k] = k < R ? wt[k] : 0.0f;
    dk[k] = slot_ok(rk[k], rows_in) ? rk[k] / cap : -1;
  }
  const int n16 = H / 8;
  const u32x4* ybase = (const u32x4*)y;
  for (int base = part * kWave * V; base < n16; base += W * kWave * V) {
    RowRegs<V> v[kPresumMaxR];
#pragma unroll
    for (int k = 0; k < kPresumMaxR; ++k)
      if (dk[k] >= 0) load_row16(v[k], ybase + (size_t)rk[k] * n16, base, n16);
#pragma unroll
    for (int k0 = 0; k0 < kPresumMaxR; ++k0) {
      if (dk[k0] < 0) continue;
      bool leader = true;
#pragma unroll
      for (int k2 = 0; k2 < k0; ++k2) leader = leader && dk[k2] != dk[k0];
      if (!leader) continue;
      float acc[V][8];
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
#pragma unroll
      for (int k = k0; k < kPresumMaxR; ++k)
        if (dk[k] == dk[k0]) fma_row(acc, v[k], wk[k]);
      store_acc(acc, (u32x4*)(partial + ((size_t)tok * R + k0) * H), base, n16);
    }
  }
}

// Source side: out = bf16( sum over leaders, k order, of float(partial) ),
// from 0 (a fused multiply-add by 1 is an exact add). Two rows in flight.
__global__ __launch_bounds__(kBlock) void presum_final_kernel(const uint16_t* partial,
                                                              const int32_t* comb_row,
                                                              uint16_t* out, int NT, int R, int H,
                                                              int cap, int64_t rows_in) {
  const int wv = wave_index();
  const int tok = wv / kCombWaves;
  const int part = wv % kCombWaves;
  if (tok >= NT) return;
  const int32_t* rows = comb_row + (size_t)tok * R;
  const int n16 = H / 8;
  const u32x4* pbase = (const u32x4*)(partial + (size_t)tok * R * H);
  u32x4* o = (u32x4*)(out + (size_t)tok * H);
  uint64_t leaders = 0;
  for (int k = 0; k < R; ++k)
    if (is_leader(rows, k, cap, rows_in)) leaders |= 1ull << k;
  for (int base = part * kWave * kCombV; base < n16; base += kCombWaves * kWave * kCombV) {
    float acc[kCombV][8];
#pragma unroll
    for (int i = 0; i < kCombV; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    uint64_t left = leaders;
    while (left) {
      const int ka = __builtin_ctzll(left);
      left &= left - 1;
      RowRegs<kCombV> va, vb;
      load_row16(va, pbase + (size_t)ka * n16, base, n16);
      const int kb = left ? __builtin_ctzll(left) : -1;
      if (kb >= 0) {
        left &= left - 1;
        load_row16(vb, pbase + (size_t)kb * n16, base, n16);
      }
      fma_row(acc, va, 1.0f);
      if (kb >= 0) fma_row(acc, vb, 1.0f);
    }
    store_acc(acc, o, base, n16);
  }
}

// Stand-in expert: one wave per delivered grouped row r of rank d; its local
// expert j is the one with grp_off[d][j] <= r < grp_off[d][j+1].
__global__ __launch_bounds__(kBlock) void expert_stub_kernel(
    const uint8_t* __restrict__ g0, const uint8_t* __restrict__ g1,
    const float* __restrict__ alpha, const int32_t* __restrict__ grp_off,
    uint16_t* __restrict__ y, int L, int H, int64_t cap, int payload) {
  const int d = blockIdx.y;
  const int r = wave_index();
  const int32_t* go = grp_off + (size_t)d * (L + 1);
  const int64_t lim = go[L] < cap ? go[L] : cap;
  if (r >= lim) return;
  int lo = 0, hi = L - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (go[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int e = d * L + lo;
  const size_t grow = (size_t)d * cap + r;
  uint16_t* yr = y + grow * H;
  const int lane = lane_id();
  if (payload == 0) {
    const u32x4* in = (const u32x4*)(g0 + grow * (size_t)H * 2);
    const float a = alpha ? alpha[e] : 1.0f;
    for (int c = lane; c < H / 8; c += kWave) {
      u32x4 v = load_stream(&in[c]);
      if (alpha) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t lo16 = f32_to_bf16_bits(bf16_lo(v[h]) * a);
          const uint32_t hi16 = f32_to_bf16_bits(bf16_hi(v[h]) * a);
          v[h] = lo16 | (hi16 << 16);
        }
      }
      store_stream(&((u32x4*)yr)[c], v);
    }
  } else {
    const u32x4* codes = (const u32x4*)(g0 + grow * (size_t)H);
    const float* scales = (const float*)(g1 + grow * (size_t)(H / 32));
    for (int c = lane; c < H / 16; c += kWave) {
      const u32x4 v = load_stream(&codes[c]);
      const float sc = scales[(c * 16) / 128];
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const uint32_t b0 = f32_to_bf16_bits(e4m3_to_f32(q[h] & 0xff) * sc);
        const uint32_t b1 = f32_to_bf16_bits(e4m3_to_f32((q[h] >> 8) & 0xff) * sc);
        const uint32_t b2 = f32_to_bf16_bits(e4m3_to_f32((q[h] >> 16) & 0xff) * sc);
        const uint32_t b3 = f32_to_bf16_bits(e4m3_to_f32(q[h] >> 24) * sc);
        o[2 * h] = b0 | (b1 << 16);
        o[2 * h + 1] = b2 | (b3 << 16);
      }
      store_stream(&((u32x4*)yr)[2 * c], u32x4{o[0], o[1], o[2], o[3]});
      store_stream(&((u32x4*)yr)[2 * c + 1], u32x4{o[4], o[5], o[6], o[7]});
    }
  }
}

unsigned blocks_for(int64_t waves) {
  return (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

}  // namespace

// Shape by token count, as measured on gfx950: at decode scale (4096 tokens)
// two waves of 7 chunks per lane per token ran 87-88 us and seven waves of 2
// chunks 88-89 us; at prefill scale (32768 tokens) the seven-wave form ran
// 696 us against 721-723 us. Both give identical bytes (same FMA order).
hipError_t launch_combine(const Dims& d, const uint16_t* y, const float* w, const PlanPtrs& p,
                          uint16_t* out, hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  const int64_t rows_in = (int64_t)d.N * d.cap;
  if (d.NT >= 16384) {
    hipLaunchKernelGGL((combine_kernel<2, 7, 2>), dim3(blocks_for(d.NT * 7)), dim3(kBlock), 0,
                       stream, y, w, p.comb_row, out, (int)d.NT, d.R, d.H, rows_in);
  } else {
    hipLaunchKernelGGL((combine_kernel<kCombV, kCombWaves, kCombRows>),
                       dim3(blocks_for(d.NT * kCombWaves)), dim3(kBlock), 0, stream, y, w,
                       p.comb_row, out, (int)d.NT, d.R, d.H, rows_in);
  }
  return hipGetLastError();
}

hipError_t launch_combine_presum(const Dims& d, const uint16_t* y, const float* w,
                                 const PlanPtrs& p, uint16_t* partial, uint16_t* out,
                                 hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  const dim3 grid(blocks_for(d.NT * kCombWaves));
  const int64_t rows_in = (int64_t)d.N * d.cap;
  if (d.R <= kPresumMaxR)
    hipLaunchKernelGGL((presum_rows_kernel<kPresumV, kPresumW>), dim3(blocks_for(d.NT * kPresumW)),
                       dim3(kBlock), 0, stream, y, w, p.comb_row, partial, (int)d.NT, d.R, d.H,
                       (int)d.cap, rows_in);
  else
    hipLaunchKernelGGL(presum_kernel, grid, dim3(kBlock), 0, stream, y, w, p.comb_row, partial,
                       (int)d.NT, d.R, d.H, (int)d.cap, rows_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(presum_final_kernel, grid, dim3(kBlock), 0, stream, partial, p.comb_row, out,
                     (int)d.NT, d.R, d.H, (int)d.cap, rows_in);
  return hipGetLastError();
}

hipError_t launch_expert_stub(const Dims& d, const void* const grouped[2], const float* alpha,
                              const PlanPtrs& p, uint16_t* y, hipStream_t stream) {
  const int64_t rows = d.cap < d.NTR ? d.cap : d.NTR;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(expert_stub_kernel, dim3(blocks_for(rows), d.N), dim3(kBlock), 0, stream,
                     (const uint8_t*)grouped[0],
                     d.planes > 1 ? (const uint8_t*)grouped[1] : nullptr, alpha, p.grp_off, y,
                     d.L, d.H, d.cap, d.payload);
  return hipGetLastError();
}

}  // namespace ep
