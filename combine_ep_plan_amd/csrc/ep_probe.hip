// Access-pattern probe: the copy, fill, read and read-mix shapes the sender,
// receiver and combine were chosen on, with the same lane loop (lane l moves
// 16-byte chunks l, l + 64, ... of its wave's piece; non-temporal stores).
// Measurement only: no step of dispatch or combine runs here.
//
// A launch walks `rows` rows (output rows; source rows for read and the
// scatters) in pieces of piece_bytes. By default wave w moves piece w and
// exits, so consecutive waves take consecutive pieces; with `waves` set,
// that many waves walk the pieces grid-stride. The XCD option renumbers
// blocks as the sender does, so XCD x takes the x-th eighth of the pieces.
//
// Modes:
//   copy: out row i, piece p = the xor of its fan_in source rows' piece p,
//         read in_flight rows at a time; the source rows come from `table`
//         (fan_in entries per row) or, without one, are rows i + j * rows
//         for input j (fan_in linear regions; one region is a plain copy);
//   fill: every piece written with a pattern, nothing read;
//   read: rows read (from `table` or in order), nothing written except, for
//         a pattern no probe input holds, one word per lane at dst (keeps the
//         loads live; dst holds 256 bytes);
//   scatter: source row i, piece p, read once and written to its fan_in
//         output rows table[i * fan_in + k] (without a table, rows
//         i * fan_in + k): the token-order sender's shape;
//   scatter-wide: the same from source rows twice as long, each output
//         chunk the xor of two adjacent source chunks (a 2:1 narrowing, as
//         the quantising sender reads bf16 and writes one byte per value).
#include "ep_device.hpp"
#include "ep_probe.hpp"

namespace ep {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeBlock = kProbeWaves * kWave;

struct ProbeArgs {
  u32x4* dst;
  const u32x4* src;
  const int32_t* table;
  int32_t rows, indexed_rows;
  int32_t row16, piece16;  // 16-byte chunks per row and per piece
  int32_t ppr;             // pieces per row
  uint32_t div_m, div_l;   // n / ppr = (mulhi(n, m) + n) >> l (Granlund-Montgomery)
  int32_t pieces;          // rows * ppr
  int32_t fan_in;          // source rows per output row (a multiple of F), or the reverse
  int32_t stride;          // waves of a grid-stride launch, 0 otherwise
  int32_t xcd, nb;         // XCD renumbering; launched blocks (a multiple of 8 with it)
  int32_t wpb;             // waves per workgroup: 1 or kProbeWaves
};

template <bool NT>
__device__ __forceinline__ u32x4 probe_load(const u32x4* p) {
  if constexpr (NT) return load_stream(p);
  else return *p;
}

// One piece w. V chunks per lane, and F of the fan_in source rows, are in
// flight per batch. The table is read-only for the launch; read through the
// constant address space, each wave-uniform entry comes by one scalar load,
// as the sender's send_slot entry does.
template <int MODE, int V, int F, bool NT>
__device__ __forceinline__ void probe_piece(const ProbeArgs& a, int w) {
  const int row = wave_uniform(
      (int)(((uint64_t)__umulhi((uint32_t)w, a.div_m) + (uint32_t)w) >> a.div_l));
  const int pc = w - row * a.ppr;
  const int64_t off = (int64_t)pc * a.piece16 + lane_id();
  const int64_t out = (int64_t)row * a.row16 + off;
  typedef const __attribute__((address_space(4))) int32_t* const_table;
  if (MODE == kProbeScatter || MODE == kProbeScatterWide) {
    constexpr int S = MODE == kProbeScatterWide ? 2 : 1;  // source chunks per output chunk
    const int64_t in = ((int64_t)row * a.row16 + off) * S;
    for (int c0 = 0; c0 < a.piece16; c0 += kWave * V) {
      u32x4 r[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int64_t c = in + (int64_t)(c0 + kWave * i) * S;
        r[i] = probe_load<NT>(&a.src[c]);
        if (S == 2) r[i] ^= probe_load<NT>(&a.src[c + 1]);
      }
      asm volatile("" ::: "memory");
      for (int k = 0; k < a.fan_in; ++k) {
        int d = a.table ? ((const_table)a.table)[(int64_t)row * a.fan_in + k]
                        : row * a.fan_in + k;
        if ((uint32_t)d >= (uint32_t)a.indexed_rows) d = 0;  // any table entry stays in bounds
        const int64_t o = (int64_t)d * a.row16 + off + c0;
#pragma unroll
        for (int i = 0; i < V; ++i) store_stream(&a.dst[o + kWave * i], r[i]);
      }
    }
    return;
  }
  if (MODE == kProbeFill) {
    const u32x4 v = {(uint32_t)w, (uint32_t)lane_id(), 0x5a5a5a5au, 0u};
    for (int c0 = 0; c0 < a.piece16; c0 += kWave * V) {
#pragma unroll
      for (int i = 0; i < V; ++i) store_stream(&a.dst[out + c0 + kWave * i], v);
    }
    return;
  }
  for (int c0 = 0; c0 < a.piece16; c0 += kWave * V) {
    u32x4 acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = u32x4{0u, 0u, 0u, 0u};
    for (int k0 = 0; k0 < a.fan_in; k0 += F) {
      u32x4 r[F][V];
#pragma unroll
      for (int j = 0; j < F; ++j) {
        const int k = k0 + j;
        int s = a.table ? ((const_table)a.table)[(int64_t)row * a.fan_in + k] : row + k * a.rows;
        if ((uint32_t)s >= (uint32_t)a.indexed_rows) s = 0;  // any table entry stays in bounds
        const int64_t in = (int64_t)s * a.row16 + off + c0;
#pragma unroll
        for (int i = 0; i < V; ++i) r[j][i] = probe_load<NT>(&a.src[in + kWave * i]);
      }
      asm volatile("" ::: "memory");  // every load of the batch above its use
#pragma unroll
      for (int j = 0; j < F; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] ^= r[j][i];
    }
    if (MODE == kProbeCopy) {
#pragma unroll
      for (int i = 0; i < V; ++i) store_stream(&a.dst[out + c0 + kWave * i], acc[i]);
    } else {
      uint32_t x = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) x ^= acc[i].x ^ acc[i].y ^ acc[i].z ^ acc[i].w;
      if (x == 0x9e3779b9u) ((uint32_t*)a.dst)[lane_id()] = x;
    }
  }
}

template <int MODE, int V, int F, bool NT>
__global__ __launch_bounds__(kProbeBlock) void probe_pattern_kernel(ProbeArgs a) {
  int b = blockIdx.x;
  if (a.xcd) b = (b & 7) * (a.nb >> 3) + (b >> 3);
  const int first = b * a.wpb + wave_uniform((int)threadIdx.x / kWave);
  if (a.stride == 0) {
    if (first < a.pieces) probe_piece<MODE, V, F, NT>(a, first);
    return;
  }
  if (first >= a.stride) return;  // the last block's spare waves
  for (int w = first; w < a.pieces; w += a.stride) probe_piece<MODE, V, F, NT>(a, w);
}

template <int MODE, int V, int F>
hipError_t launch_v(const ProbeArgs& a, bool nt, hipStream_t stream) {
  const dim3 grid((unsigned)a.nb), block((unsigned)(a.wpb * kWave));
  if constexpr (MODE == kProbeFill) {
    hipLaunchKernelGGL((probe_pattern_kernel<MODE, V, F, false>), grid, block, 0, stream, a);
  } else {
    if (nt)
      hipLaunchKernelGGL((probe_pattern_kernel<MODE, V, F, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((probe_pattern_kernel<MODE, V, F, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

template <int MODE, int F>
hipError_t launch_f(const ProbeArgs& a, int v, bool nt, hipStream_t stream) {
  switch (v) {
    case 1: return launch_v<MODE, 1, F>(a, nt, stream);
    case 2: return launch_v<MODE, 2, F>(a, nt, stream);
    case 4: if constexpr (F <= 4) return launch_v<MODE, 4, F>(a, nt, stream); break;
    case 7: if constexpr (F <= 2) return launch_v<MODE, 7, F>(a, nt, stream); break;
    case 14: if constexpr (F == 1) return launch_v<MODE, 14, F>(a, nt, stream); break;
    case 16: if constexpr (F == 1) return launch_v<MODE, 16, F>(a, nt, stream); break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

int probe_inflight(int piece_bytes, int in_flight) {
  if (piece_bytes <= 0 || piece_bytes % 1024 != 0) return 0;
  const int per_lane = piece_bytes / 1024;  // 16-byte chunks per lane in a piece
  for (int v : {16, 14, 7, 4, 2, 1})
    if (v * in_flight <= 16 && per_lane % v == 0) return v;
  return 0;
}

hipError_t launch_probe_pattern(const ProbeShape& s, hipStream_t stream) {
  ProbeArgs a{};
  a.dst = (u32x4*)s.dst;
  a.src = (const u32x4*)s.src;
  a.table = s.table;
  a.fan_in = s.fan_in;
  a.rows = s.rows;
  a.indexed_rows = s.indexed_rows;
  a.row16 = s.row_bytes / 16;
  a.piece16 = s.piece_bytes / 16;
  a.ppr = s.row_bytes / s.piece_bytes;
  uint32_t l = 0;
  while ((1u << l) < (uint32_t)a.ppr) ++l;
  a.div_l = l;
  a.div_m = (uint32_t)(((((uint64_t)1 << l) - (uint64_t)a.ppr) << 32) / (uint64_t)a.ppr + 1);
  a.pieces = s.rows * a.ppr;
  if (a.pieces == 0) return hipSuccess;
  const int64_t waves = s.waves > 0 ? s.waves : a.pieces;
  a.stride = s.waves > 0 ? s.waves : 0;
  a.wpb = s.one_wave ? 1 : kProbeWaves;
  int64_t nb = (waves + a.wpb - 1) / a.wpb;
  a.xcd = s.xcd ? 1 : 0;
  if (s.xcd) nb = (nb + 7) / 8 * 8;
  a.nb = (int32_t)nb;
  const int v = probe_inflight(s.piece_bytes, s.mode == kProbeScatterWide ? 2 : s.in_flight);
  switch (s.mode) {
    case kProbeFill: return launch_f<kProbeFill, 1>(a, v, false, stream);
    case kProbeRead: return launch_f<kProbeRead, 1>(a, v, s.nt_loads, stream);
    case kProbeScatter: return launch_f<kProbeScatter, 1>(a, v, s.nt_loads, stream);
    case kProbeScatterWide: return launch_f<kProbeScatterWide, 1>(a, v, s.nt_loads, stream);
    case kProbeCopy:
      switch (s.in_flight) {
        case 1: return launch_f<kProbeCopy, 1>(a, v, s.nt_loads, stream);
        case 2: return launch_f<kProbeCopy, 2>(a, v, s.nt_loads, stream);
        case 4: return launch_f<kProbeCopy, 4>(a, v, s.nt_loads, stream);
        case 8: return launch_f<kProbeCopy, 8>(a, v, s.nt_loads, stream);
        default: break;
      }
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

}  // namespace ep
