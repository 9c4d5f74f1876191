// nvfp4_encode.h -- NVFP4 encoding of 16-element groups, shared by the two
// cache writers (msa_nvfp4_quantize and msa_qkv_rope_insert). Format:
// NVFP4 as reproduced by the pages' 34,560 bytes per token (MiniMax-M3.1-Flash
// lands in vLLM on day one, first paragraph).
#pragma once

#include "nvfp4_tile.h"

namespace msa {

// NVFP4 encoding of one 16-element group x[0..15] (fp32), given the scale
// bounds (ScaleBounds, e.g. staged in LDS). Every decision is an exact fp32
// comparison, so no division or rounding enters one:
//   - scale byte: the E4M3 value nearest to amax / 6 (ties to even,
//     satfinite). The hardware conversion of amax * (1/6), rounded in fp32,
//     lands at most one byte c off the exact answer (its relative error,
//     2^-23, is far below the 2^-4 between neighbouring midpoints); amax is
//     then compared with the bounds of c (6 x its two midpoints) and moves
//     to the neighbour it exceeds, a tie going to the even byte;
//   - codes: the E2M1 magnitude nearest to |x| / s (ties to even) is the
//     number of the seven midpoints s x {1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5}
//     that |x| passes, counting equality for the midpoints whose upper
//     neighbour is the even code (the 2nd, 4th and 6th); with a zero scale
//     every code is zero (only the sign bit is kept).
// Element i's nibble (sign bit 3) goes to bits 4 (i % 8) of packed[i / 8]
// (channel 2j in the low nibble of byte j). Returns the scale byte.
__device__ __forceinline__ int nvfp4_encode_group(const float (&x)[16], const float* bnd,
                                                  uint32_t (&packed)[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float q = fminf(amax * (1.0f / 6.0f), 448.0f);
  const int c = __builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0x7F;
  const float lo = bnd[c], hi = bnd[c + 1];
  const int odd = c & 1;
  const int sb = c + ((amax > hi || (amax == hi && odd)) ? 1 : 0) -
                 ((amax < lo || (amax == lo && odd)) ? 1 : 0);
  const float s = sb ? __builtin_amdgcn_cvt_f32_fp8(sb, 0) : __builtin_huge_valf();
  const float m0 = 0.25f * s, m1 = 0.75f * s, m2 = 1.25f * s, m3 = 1.75f * s;
  const float m4 = 2.5f * s, m5 = 3.5f * s, m6 = 5.0f * s;
  packed[0] = packed[1] = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = fabsf(x[i]);
    uint32_t nib = (__float_as_uint(x[i]) >> 28) & 8u;
    nib += a > m0;
    nib += a >= m1;
    nib += a > m2;
    nib += a >= m3;
    nib += a > m4;
    nib += a >= m5;
    nib += a > m6;
    packed[i >> 3] |= nib << (4 * (i & 7));
  }
  return sb;
}

}  // namespace msa
