// Dispatch sender with block-fp8 quantisation fused in.
//
// Method: "Enabling trillion-parameter models on AWS EFA", section
// "Evaluation": dispatch moves block-scaled fp8 rows (the DeepSeek-V3 /
// Kimi-K2 setting), combine moves bf16. Here the sender reads each bf16 token
// row once, quantises it per block of 128 values (scale = amax / 448, codes =
// OCP e4m3fn of x / scale, nearest even, clamped to +-448) and writes the code
// and scale rows to the token's R send slots, so the send buffer holds half
// the bytes of a bf16 dispatch.
//
// One wave per 1024-value segment of a token row. Lane l holds 16-byte chunks
// l and l+64 of the segment (8 bf16 each); the 16 lanes 16g .. 16g+15 of one
// step hold one 128-value block, so the block's amax is a reduction over one
// DPP row. The scale is the IEEE fp32 division amax / 448. The codes are
// those of the IEEE fp32 quotient x / scale (the operation a CPU reference
// performs), obtained without a division per value (quantise_step).
#include "ep_device.hpp"
#include "ep_kernels.hpp"
#include "ep_plan_device.hpp"

namespace ep {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWavesPerBlock * kWave;
// Segment per wave: 2 chunks of 8 bf16 per lane, 128 chunks = 1024 values =
// 8 scale blocks. Small segments keep the kernel at ~40 VGPRs, so 8 waves per
// SIMD overlap one wave's loads with another's R-fold stores; one wave per
// whole 7168-value token (256 VGPRs, one wave per SIMD) ran 1.5x slower.
constexpr int kQV = 2;
constexpr int kQSeg = kWave * kQV;
constexpr int kQBlocks = kQSeg / 16;

__device__ __forceinline__ int wave_index() {
  return wave_uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
}

// A send position the whole wave reads (its index is wave-uniform), taken
// through the constant address space so that it comes by a scalar load. The
// plan wrote the table in an earlier launch; this one only reads it. With a
// vector load, the wait for the entry also waits for the wave's earlier row
// stores, which the same counter tracks on gfx950, so a token's R rows went
// out one after the other.
__device__ __forceinline__ int send_pos_at(const int32_t* send_pos, size_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)send_pos)[i];
}

// OCP e4m3fn code of q (|q| <= 448), round to nearest, ties to even. For
// |q| >= 2^-6 with 2^E <= |q| < 2^(E+1): N = rne(|q| * 2^(3-E)) in [8, 16],
// code = (E + 6) * 8 + N (N = 16 carries into the next exponent). Below 2^-6
// (subnormals): code = rne(|q| * 2^9) in [0, 8]. Both scalings are by powers
// of two, so exact.
__device__ __forceinline__ uint32_t f32_to_e4m3(float q) {
  const uint32_t bits = __float_as_uint(q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const int E = (int)((bits >> 23) & 0xffu) - 127;
    const float scaled = a * __uint_as_float((uint32_t)(127 + 3 - E) << 23);
    code = (uint32_t)((E + 6) * 8) + (uint32_t)__builtin_rintf(scaled);
  }
  return sign | code;
}

// Codes and scale of one step (8 values per lane, 16 lanes per block).
//
// Fast path: y = 1 / scale once per block (IEEE division), then per value
// q0 = |x| y and one correction q = q0 + (|x| - scale q0) y (two FMAs; the
// residual is exact), clamped to 448, signed by x, and encoded by the
// hardware conversion, which equals f32_to_e4m3 on every |q| <= 448
// (tests/test_gpu_fp8_convert.py checks every such fp32 value). For a
// bf16 x and a bf16 block amax of at least 2^-96 this q gives the same e4m3
// code as the IEEE quotient x / scale: checked for every such pair (524.8 M
// of them) by tests/test_fp8_reciprocal.py, which runs these same operations
// on the CPU. Everything else takes the exact path below for the whole wave:
// a smaller nonzero amax, an infinite amax, or a NaN anywhere in the step.
//
// Exact path: amax with NaN left out (a NaN never compares greater; an
// infinite value makes amax and the scale infinite), IEEE division per
// value, the software encoder; a NaN quotient (a NaN value, or an infinite
// one over its infinite scale) is the NaN code 0x7F, kept from the clamp,
// which would turn it into -448.
__device__ __forceinline__ void quantise_step(const u32x4& r, uint32_t packed[2], float& scale_out) {
  float v[8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = bf16_lo(r[h]);
    v[2 * h + 1] = bf16_hi(r[h]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  // Over the block's 16 lanes (one DPP row): the maximum of non-negative
  // floats is the maximum of their bit patterns, and a NaN stays the largest.
  uint32_t ab = __float_as_uint(amax);
  ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ab, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ab, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ab, 0x141, 0xF, 0xF, false));  // half-row mirror
  ab = max(ab, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ab, 0x140, 0xF, 0xF, false));  // row mirror
  amax = __uint_as_float(ab);
  float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
  const float y = 1.0f / scale;
  uint32_t qmax = 0;
  float q[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float a = fabsf(v[j]);
    const float q0 = a * y;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-scale, q0, a), y, q0);
    qmax = max(qmax, __float_as_uint(q1));
    q[j] = __builtin_copysignf(fminf(q1, 448.0f), v[j]);
  }
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[4], q[5], 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(q[6], q[7], w1, true);
  packed[0] = (uint32_t)w0;
  packed[1] = (uint32_t)w1;
  const bool exact = (amax > 0.0f && amax < 0x1p-96f) || !(amax < __builtin_inff()) ||
                     qmax > 0x7f800000u;
  if (ballot(exact)) {  // wave-uniform: the shuffles below need every lane
    amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(v[j]);
      amax = a > amax ? a : amax;
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float qq = v[j] / scale;
      c[j] = __builtin_isnan(qq) ? 0x7Fu : f32_to_e4m3(fminf(fmaxf(qq, -448.0f), 448.0f));
    }
    packed[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    packed[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
  }
  scale_out = scale;
}

// The sender's work for wave w (token w / nseg, segment w % nseg). With
// ROW_SCALES the wave also writes its blocks' scales to the R send rows;
// otherwise it leaves them in tok_scale (LDS, indexed by block) for the
// workgroup to write whole scale rows.
template <bool ROW_SCALES>
__device__ __forceinline__ void quant_wave(int w, const uint16_t* __restrict__ x,
                                           uint8_t* __restrict__ codes, float* __restrict__ scales,
                                           const int32_t* __restrict__ send_pos, int NT, int T,
                                           int R, int H, int nseg, float* tok_scale) {
  const int tok = wave_uniform(w / nseg);
  if (tok >= NT) return;
  const int lane = lane_id();
  const int n16 = H / 8;
  const int nblk = H / 128;
  const int TR = T * R;
  const int s = tok / T;
  const int base = (w - tok * nseg) * kQSeg;
  const u32x4* src = (const u32x4*)(x + (size_t)tok * H);
  RowRegs<kQV> r;
  // Cached loads: 53 vs 58 us with non-temporal ones on the decode-shape fp8
  // workload (the senders all read their token rows this way).
  load_row16<kQV, false>(r, src, base, n16);
  uint32_t packed[kQV][2];
  float sc[kQV];
#pragma unroll
  for (int i = 0; i < kQV; ++i) quantise_step(r.v[i], packed[i], sc[i]);
  // Lane b < kQBlocks collects the scale of block b of this segment: block b
  // was computed in step b / 4 by lane group b % 4.
  float my_scale = 0.0f;
#pragma unroll
  for (int i = 0; i < kQV; ++i) {
    const float t = __shfl(sc[i], 16 * (lane % 4));
    if (lane / 4 == i) my_scale = t;
  }
  const int blk0 = base / 16;
  const int seg_blocks = nblk - blk0 < kQBlocks ? nblk - blk0 : kQBlocks;
  if (!ROW_SCALES && lane < seg_blocks) tok_scale[blk0 + lane] = my_scale;
  for (int k = 0; k < R; ++k) {
    const int p = send_pos_at(send_pos, (size_t)tok * R + k);
    if (p < 0 || p >= TR) continue;
    const size_t row = (size_t)s * TR + p;
    uint64_t* crow = (uint64_t*)(codes + row * H);  // 8 codes per chunk
#pragma unroll
    for (int i = 0; i < kQV; ++i) {
      const int c = base + lane + kWave * i;
      if (c < n16)
        __builtin_nontemporal_store((uint64_t)packed[i][0] | ((uint64_t)packed[i][1] << 32),
                                    &crow[c]);
    }
    if (ROW_SCALES && lane < seg_blocks)
      __builtin_nontemporal_store(my_scale, &scales[row * nblk + blk0 + lane]);
  }
}

// One workgroup of kTokWaves waves per token (H <= kTokWaves * 1024): the
// waves quantise their segments and write the codes, then the token's whole
// scale row (4 H / 128 bytes) goes to each of its R send rows in one store.
// Scale rows written in 32-byte pieces by separate waves cost ~10% of the
// sender's time (51 vs 46 us at decode shapes with the scale stores left
// out); with whole rows the decode-shape dispatch + combine step took 226 us
// against 232 us (prefill shapes: unchanged).
constexpr int kTokThreads = 512;
constexpr int kTokWaves = kTokThreads / kWave;

template <bool EXCHANGE>
__global__ __launch_bounds__(kTokThreads) void pack_quant_tok_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, float* __restrict__ scales,
    PlanPtrs p, int NT, int N, int E, int L, int T, int R, int H, int nseg, int64_t cap,
    int32_t* status) {
  __shared__ float tok_scale[kTokWaves * kQBlocks];
  extern __shared__ int32_t lds[];
  int b = blockIdx.x;
  if (EXCHANGE) {
    if (b < N) {  // block-uniform: the count exchange (see pack_exchange_kernel)
      exchange_block<kTokThreads>(b, 0, b, N, N, E, L, (int64_t)T * R, cap, p, status, lds);
      return;
    }
    b -= N;
  }
  const int tok = b;
  if (tok >= NT) return;  // block-uniform
  const int wv = (int)threadIdx.x / kWave;
  if (wv < nseg)
    quant_wave<false>(tok * nseg + wv, x, codes, scales, p.send_pos, NT, T, R, H, nseg, tok_scale);
  __syncthreads();
  const int lane = lane_id();
  const int nblk = H / 128;
  const int TR = T * R;
  const int s = tok / T;
  for (int k = wave_uniform(wv); k < R; k += kTokWaves) {
    const int pos = send_pos_at(p.send_pos, (size_t)tok * R + k);
    if (pos < 0 || pos >= TR) continue;
    if (lane < nblk)
      __builtin_nontemporal_store(tok_scale[lane], &scales[((size_t)s * TR + pos) * nblk + lane]);
  }
}

__global__ __launch_bounds__(kBlock) void pack_quant_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, float* __restrict__ scales,
    const int32_t* __restrict__ send_pos, int NT, int T, int R, int H, int nseg) {
  quant_wave<true>(wave_index(), x, codes, scales, send_pos, NT, T, R, H, nseg, nullptr);
}

// As pack_quant_kernel, with the count exchange done by the first N blocks
// (see pack_exchange_kernel): for sources whose slots fit one plan chunk.
__global__ __launch_bounds__(kBlock) void pack_quant_exchange_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ codes, float* __restrict__ scales,
    PlanPtrs p, int N, int E, int L, int T, int R, int H, int nseg, int64_t cap,
    int32_t* status) {
  extern __shared__ int32_t lds[];
  const int b = blockIdx.x;
  if (b < N) {  // block-uniform
    exchange_block<kBlock>(b, 0, b, N, N, E, L, (int64_t)T * R, cap, p, status, lds);
    return;
  }
  const int w = wave_uniform((b - N) * kWavesPerBlock + (int)threadIdx.x / kWave);
  quant_wave<true>(w, x, codes, scales, p.send_pos, N * T, T, R, H, nseg, nullptr);
}

}  // namespace

hipError_t launch_pack_quant(const Dims& d, const uint16_t* x, const PlanPtrs& p,
                             void* const send[2], hipStream_t stream) {
  if (d.NT == 0) return hipSuccess;
  const int nseg = (d.H / 8 + kQSeg - 1) / kQSeg;
  if (nseg <= kTokWaves) {
    hipLaunchKernelGGL(pack_quant_tok_kernel<false>, dim3((unsigned)d.NT), dim3(kTokThreads), 0,
                       stream, x, (uint8_t*)send[0], (float*)send[1], p, (int)d.NT, d.N, d.E,
                       d.L, d.T, d.R, d.H, nseg, d.cap, (int32_t*)nullptr);
    return hipGetLastError();
  }
  const int64_t waves = d.NT * nseg;
  hipLaunchKernelGGL(pack_quant_kernel, dim3((unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock)),
                     dim3(kBlock), 0, stream, x, (uint8_t*)send[0], (float*)send[1], p.send_pos,
                     (int)d.NT, d.T, d.R, d.H, nseg);
  return hipGetLastError();
}

hipError_t launch_dispatch_quant(const Dims& d, const int32_t* idx, const uint16_t* x,
                                 const PlanPtrs& p, void* const send[2], void* const grouped[2],
                                 int32_t* status, hipStream_t stream) {
  if (!dispatch_fused_fits(d) || d.NT == 0) {
    hipError_t e = launch_plan(d, idx, p, status, stream, false);
    if (e == hipSuccess) e = launch_pack_quant(d, x, p, send, stream);
    if (e == hipSuccess) e = launch_recv(d, send, p, grouped, stream);
    return e;
  }
  hipError_t e = launch_plan_local(d, idx, p, status, stream, false);
  if (e != hipSuccess) return e;
  const int nseg = (d.H / 8 + kQSeg - 1) / kQSeg;
  if (nseg <= kTokWaves) {
    hipLaunchKernelGGL(pack_quant_tok_kernel<true>, dim3((unsigned)(d.N + d.NT)),
                       dim3(kTokThreads), lds_exchange_bytes(d, kTokThreads), stream, x,
                       (uint8_t*)send[0], (float*)send[1], p, (int)d.NT, d.N, d.E, d.L, d.T, d.R,
                       d.H, nseg, d.cap, status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_recv(d, send, p, grouped, stream);
  }
  const int64_t waves = d.NT * nseg;
  const unsigned grid = (unsigned)d.N + (unsigned)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(pack_quant_exchange_kernel, dim3(grid), dim3(kBlock),
                     lds_exchange_bytes(d, kBlock),
                     stream, x, (uint8_t*)send[0], (float*)send[1], p, d.N, d.E, d.L, d.T, d.R,
                     d.H, nseg, d.cap, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_recv(d, send, p, grouped, stream);
}

}  // namespace ep
