// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
// Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC 2011), written
// from its published definition, and the draws the random gate options
// take from it.
//
// One round on the counter (c0, c1, c2, c3) with key (k0, k1): with the
// 64-bit products M0*c0 = (hi0, lo0) and M1*c2 = (hi1, lo1), the new counter
// is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by the Weyl
// increments between rounds; ten rounds.
//
// Draw n of stream s under a 64-bit seed: word n % 4 of the block at counter
// (n / 4 low 32 bits, n / 4 high 32 bits, s, 0) with key (seed low, seed
// high).  A word w gives the fp32 uniform ((w >> 9) + 0.5) * 2^-23, exactly
// representable and inside (0, 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint32_t lo0 = kPhiloxM0 * c.x, hi0 = __umulhi(kPhiloxM0, c.x);
    const uint32_t lo1 = kPhiloxM1 * c.z, hi1 = __umulhi(kPhiloxM1, c.z);
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// The four words of block b of a stream.
__device__ __forceinline__ uint4 philox_block(uint32_t seed_lo, uint32_t seed_hi, uint32_t stream, uint64_t b) {
  return philox4x32_10(make_uint4((uint32_t)b, (uint32_t)(b >> 32), stream, 0u), seed_lo, seed_hi);
}

__device__ __forceinline__ uint32_t philox_draw(uint32_t seed_lo, uint32_t seed_hi, uint32_t stream, uint64_t n) {
  const uint4 w = philox_block(seed_lo, seed_hi, stream, n >> 2);
  const uint32_t j = (uint32_t)(n & 3);
  return j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
}

__device__ __forceinline__ float philox_uniform(uint32_t w) {
  return ((float)(w >> 9) + 0.5f) * 0x1p-23f;
}

// Streams of the random gate options.
enum { kStreamJitter = 0, kStreamRSample = 1, kStreamSecond = 2, kStreamRts = 3 };

}  // namespace moe
