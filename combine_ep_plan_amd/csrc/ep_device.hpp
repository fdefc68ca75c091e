// Device helpers for the gfx950 dispatch/combine kernels: wave64 ballot
// primitives, number-format conversions written from their definitions, and
// wave-wide 16-byte row copies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

// Status bits (mirrors EP_STATUS_* of the public header).
constexpr int kStatusBadExpert = 1;
constexpr int kStatusCapacity = 2;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Make a value that is equal on all lanes live in a scalar register.
__device__ __forceinline__ int wave_uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanes_below() {
  return (1ull << __lane_id()) - 1ull;
}

// Lanes of this wave (among `active`) holding the same `key`, built from one
// ballot per key bit: a lane matches when it agrees with us on every bit.
__device__ __forceinline__ uint64_t match_key(int key, int nbits, bool active) {
  uint64_t peers = ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t ones = ballot(active && bit);
    peers &= bit ? ones : ~ones;
  }
  return peers;
}

// float -> bf16 bits, round to nearest, ties to even (IEEE-754 binary32 with
// the low 16 fraction bits rounded away). NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u | ((u >> 16) & 0x8000u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// OCP e4m3fn code -> float: 1 sign, 4 exponent bits (bias 7), 3 fraction
// bits, no infinities, S.1111.111 = NaN, exponent 0 = subnormal m/8 * 2^-6.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t ex = (c >> 3) & 0xfu;
  const uint32_t m = c & 7u;
  float v;
  if ((c & 0x7fu) == 0x7fu) {
    v = __uint_as_float(0x7fc00000u);
  } else if (ex == 0) {
    v = (float)m * 0.001953125f;  // m * 2^-9, exact
  } else {
    v = __uint_as_float(((ex + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(ex-7)
  }
  return __uint_as_float(__float_as_uint(v) | sign);
}

// ---------------------------------------------------------------------------
// Row copies. A wave moves one row of n16 16-byte chunks: lane l handles
// chunks l, l + 64, ... V chunks per lane are loaded before any is stored so
// that a whole row is in flight at once. Callers must pass matching `base`
// and `n16` to the load and the store of a chunk set (the clamping of both
// relies on it).
//
// Row data is touched once per kernel, so loads and stores are
// non-temporal. Measured on gfx950: a wave that issues its 14 row stores back
// to back with default stores makes the L2 fetch and write every line twice
// (2x FETCH_SIZE and WRITE_SIZE against a plain copy, ~1.6x the time);
// non-temporal stores bring both back to 1x and the copy to the device's
// copy bandwidth.
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct RowRegs {
  u32x4 v[V];
};

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ void store_stream(u32x4* p, u32x4 v) {
  __builtin_nontemporal_store(v, p);
}

// Loads are unconditional: a lane past the end re-reads the row's last
// chunk (clamped index, always in bounds), so no branch separates the loads
// and all V of them are in flight together. Requires n16 >= 1. NT selects
// non-temporal loads (the default) or ordinary cached ones.
template <int V, bool NT = true>
__device__ __forceinline__ void load_row16(RowRegs<V>& r, const u32x4* src, int base, int n16) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c = base + lane + kWave * i;
    const u32x4* q = &src[c < n16 ? c : n16 - 1];
    r.v[i] = NT ? load_stream(q) : *q;
  }
  // Compiler memory barrier: keeps every load above the caller's stores
  // (otherwise each load is sunk next to its store and the row's loads
  // no longer overlap). Emits no instruction.
  asm volatile("" ::: "memory");
}

// Stores use the same clamped index: a lane past the end writes the last
// chunk, holding exactly the bytes the lane that owns that chunk writes, so
// the duplicate store is harmless and no branch is needed.
template <int V>
__device__ __forceinline__ void store_row16(const RowRegs<V>& r, u32x4* dst, int base, int n16) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int c = base + lane + kWave * i;
    store_stream(&dst[c < n16 ? c : n16 - 1], r.v[i]);
  }
}

// Fallback for rows whose size is a multiple of 4 bytes but not of 16.
__device__ __forceinline__ void copy_row4(const uint32_t* src, uint32_t* dst, int64_t n4) {
  for (int64_t c = lane_id(); c < n4; c += kWave)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[c]), &dst[c]);
}

}  // namespace ep
