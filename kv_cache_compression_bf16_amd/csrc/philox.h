// Keyformer's Gumbel noise on the device: Philox4x32-10 words and the
// Gumbel(0,1) transform in log2 units, shared by the prompt-phase scoring
// passes and the decode step.
#pragma once

#include "common.h"

namespace kvc {

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of the
// multiply-high/low S-box on words 0 and 2 with the key bumped by the Weyl
// constants between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x.z;
    // each three-way xor is one v_bitop3_b32 (truth table 0x96 = a ^ b ^ c)
    u32x4 y;
    y.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), x.y, k0, 0x96);
    y.y = (uint32_t)p1;
    y.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), x.w, k1, 0x96);
    y.w = (uint32_t)p0;
    x = y;
  }
  return x;
}

// Gumbel(0,1) noise from one 32-bit word, in log2 units: u = (2*(X>>9)+1) * 2^-24
// (exact in fp32) and zeta * log2(e) = -log2(-ln u) = -log2(-log2 u) - log2(ln 2).
// The hardware log2 is within 1.2e-7 relative of the exact value on every u of
// this grid, u -> 1 included, so the noise is good to about 1e-6 absolute.
__device__ __forceinline__ float gumbel_log2_from_word(uint32_t x) {
  const float u = (float)(((x >> 9) << 1) | 1u) * 0x1p-24f;
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u)) + 0.52876637f;
}

}  // namespace kvc
