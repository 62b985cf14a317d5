// Counter-based Philox4x32-10 for the verify kernels (device side).
//
// Definition: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3" (SC'11).  Ten rounds of
//   (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
// with the key advanced by the Weyl increments (W0, W1) before every round
// after the first.  Each 32x32->64 product is one v_mad_u64_u32 and each
// three-way XOR one v_bitop3_b32 (truth table 0x96), both close to the full
// VALU rate on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsv {

struct PhiloxOut {
  uint32_t w[4];
};

__device__ __forceinline__ PhiloxOut philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                   uint32_t k0, uint32_t k1) {
  constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
  constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t a = (uint64_t)kM0 * c0;
    const uint64_t b = (uint64_t)kM1 * c2;
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(b >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(a >> 32), c3, k1, 0x96);
    c0 = n0;
    c1 = (uint32_t)b;
    c2 = n2;
    c3 = (uint32_t)a;
    k0 += kW0;
    k1 += kW1;
  }
  PhiloxOut o;
  o.w[0] = c0;
  o.w[1] = c1;
  o.w[2] = c2;
  o.w[3] = c3;
  return o;
}

// Accept uniform of request b, position j: top 24 bits of word 0 of counter
// (0, j, b, 0), scaled to [0, 1).  Exact in fp32 and in fp64.
__device__ __forceinline__ double accept_uniform(uint64_t seed, int32_t b, int32_t j) {
  const PhiloxOut o = philox4x32_10(0u, (uint32_t)j, (uint32_t)b, 0u, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (double)(o.w[0] >> 8) * 0x1p-24;
}

// U_x = ((w >> 9) + 1/2) 2^-23, exactly: the bit pattern 0x3F800000 | (w >> 9)
// is the float 1 + (w >> 9) 2^-23 (one v_alignbit_b32 funnels the 23 bits
// under the exponent of 1.0), and subtracting 1 - 2^-24 from a float in
// [1, 2) is exact (Sterbenz), leaving (w >> 9) 2^-23 + 2^-24.
__device__ __forceinline__ float race_uniform_f32(uint32_t w) {
  const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  return f - 0x1.fffffep-1f;
}

}  // namespace rsv
