// nvfp4_encode.h -- NVFP4 encoding of 16-element groups, shared by the two
// cache writers (msa_nvfp4_quantize and msa_qkv_rope_insert). Format:
// NVFP4 as reproduced by the pages' 34,560 bytes per token (MiniMax-M3.1-Flash
// lands in vLLM on day one, first paragraph).
#pragma once

#include "nvfp4_tile.h"

namespace msa {

// NVFP4 encoding of one 16-element group x[0..15] (fp32), given the scale
// thresholds (ScaleThresholds, e.g. staged in LDS): the scale byte is the
// E4M3 value nearest to amax / 6 (ties to even, satfinite), found as the
// number of thresholds strictly below amax; each code is the E2M1 magnitude
// nearest to |x| / s (ties to even) with the sign bit of x, found by
// comparing |x| with s x the E2M1 midpoints (a binary search over the seven). Every threshold and product is
// exact in fp32, so no division or rounding enters a decision. Element i's
// nibble goes to bits 4 (i % 8) of packed[i / 8] (channel 2j in the low
// nibble of byte j). Returns the scale byte.
__device__ __forceinline__ int nvfp4_encode_group(const float (&x)[16], const float* thr,
                                                  uint32_t (&packed)[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int sb = 0;
#pragma unroll
  for (int step = 64; step > 0; step >>= 1)
    if (thr[sb + step - 1] < amax) sb += step;
  if (sb < 126 && amax == thr[sb] && (sb & 1)) sb += 1;
  const float s = e4m3_to_float(sb);
  const float m0 = 0.25f * s, m1 = 0.75f * s, m2 = 1.25f * s, m3 = 1.75f * s;
  const float m4 = 2.5f * s, m5 = 3.5f * s, m6 = 5.0f * s;
  packed[0] = packed[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = fabsf(x[i]);
    // the number of midpoints strictly below a, by a three-level binary
    // search; `upper` is the smallest midpoint >= a (the last one a did not
    // exceed), which decides a tie
    const bool g3 = a > m3;
    const float t1 = g3 ? m5 : m1;
    const bool g1 = a > t1;
    const float t0 = g3 ? (g1 ? m6 : m4) : (g1 ? m2 : m0);
    const bool g0 = a > t0;
    int mag = (g3 ? 4 : 0) + (g1 ? 2 : 0) + (g0 ? 1 : 0);
    const float upper = !g0 ? t0 : !g1 ? t1 : !g3 ? m3 : __builtin_huge_valf();
    mag += (a == upper && (mag & 1)) ? 1 : 0;  // a tie goes to the even code
    if (sb == 0) mag = 0;
    const uint32_t nib = (uint32_t(__float_as_uint(x[i]) >> 31) << 3) | uint32_t(mag);
    packed[i >> 3] |= nib << (4 * (i & 7));
  }
  return sb;
}

}  // namespace msa
