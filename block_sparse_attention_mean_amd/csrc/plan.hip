// SIP / top-k sampling plan (placeholder until the plan kernel lands).
#include "common.h"

namespace bsa {

// SplitMix64 (Steele, Lea and Flood 2014): output `i` of the stream seeded
// with `seed`, then the 44-bit fixed-point sampling offset of that row.
__host__ __device__ inline uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t sampling_offset(uint64_t seed, uint64_t row) {
  const uint64_t x = splitmix64_at(seed, row) >> 20;  // 44 bits
  const unsigned __int128 p = (unsigned __int128)x * ((1ull << 44) - (1ull << 16));
  return (uint64_t)(p >> 44);
}

int launch_sip_plan(const float *, int, int, int, int, int, uint64_t, const uint64_t *,
                    int32_t *, float *, int32_t *, double *, hipStream_t) {
  return BSA_ERR_UNSUPPORTED;
}

}  // namespace bsa
