// Test helper (not part of the library): the hardware f32 -> e4m3 pair
// conversion of gfx950 against the e4m3 rounding formula, for every fp32
// value of magnitude at most 448, both signs, both halves of the packed
// result. The quantising sender relies on the two being equal there (it
// clamps to 448 first). The formula: for 2^E <= |q| < 2^(E+1), |q| >= 2^-6,
// code = (E + 6) * 8 + rne(|q| * 2^(3 - E)); below 2^-6 (subnormal),
// code = rne(|q| * 2^9); sign in bit 7 (OCP e4m3fn, bias 7, no infinity).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ uint32_t formula_e4m3(float q) {
  const uint32_t bits = __float_as_uint(q);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const int e = (int)((bits >> 23) & 0xffu) - 127;
  return sign | ((uint32_t)((e + 6) * 8) +
                 (uint32_t)__builtin_rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23)));
}

// Thread i checks the magnitudes with bit patterns i, i + stride, ... up to
// `last` (0x43E00000 is 448): +x and -x in both word halves.
__global__ __launch_bounds__(256) void check_kernel(uint32_t last, unsigned long long* checked,
                                                    unsigned long long* bad, uint32_t* first_bad) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  unsigned long long n = 0, nbad = 0;
  for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u <= last; u += stride) {
    const float p = __uint_as_float((uint32_t)u);
    const float m = __uint_as_float((uint32_t)u | 0x80000000u);
    const uint32_t fp = formula_e4m3(p), fm = formula_e4m3(m);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p, m, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(m, p, w, true);
    n += 1;
    if ((uint32_t)w != (fp | (fm << 8) | (fm << 16) | (fp << 24))) {
      ++nbad;
      atomicMin(first_bad, (uint32_t)u);
    }
  }
  atomicAdd(checked, n);
  atomicAdd(bad, nbad);
}

}  // namespace

// counters: [checked, bad] (device, zeroed by the caller), first_bad: device
// uint32 set to 0xFFFFFFFF by the caller. Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int fp8_convert_check(void* counters, void* first_bad, hipStream_t stream) {
  unsigned long long* c = (unsigned long long*)counters;
  hipLaunchKernelGGL(check_kernel, dim3(4096), dim3(256), 0, stream, 0x43E00000u, c, c + 1,
                     (uint32_t*)first_bad);
  return (int)hipGetLastError();
}
