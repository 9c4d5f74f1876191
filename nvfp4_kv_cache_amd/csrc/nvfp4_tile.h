// nvfp4_tile.h -- shared device pieces of the HIP path: the NVFP4 -> FP8
// lookup table, the per-lane dequantiser that feeds FP8 MFMA operands, and
// small wavefront helpers.
//
// NVFP4 -> FP8: the scaled value of an E2M1 code is E2M1[m] * s for the
// block's E4M3 scale s; the query is FP8, so that product is rounded to FP8
// before the matrix multiply (MiniMax-M3.1-Flash lands in vLLM on day one,
// third paragraph). CDNA4 has no NVFP4 conversion instruction; it uses a
// small table of scaled values plus sign handling (MiniMax-M3.1-Flash
// serving summary, section "AMD uses different conversion and communication
// mechanisms"). Here the table has one 8-byte row per scale byte: byte m is
// the E4M3 encoding of E2M1[m] * s (nearest, ties to even, satfinite). A
// row lives in two dwords, so one v_perm_b32 turns four 3-bit magnitude
// indices into four FP8 magnitudes, and the sign nibble bit is OR-ed into
// bit 7.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kBlockTokens = 128;
constexpr int kGroup = 16;
constexpr int kCodeRow = kHeadDim / 2;        // 64 code bytes per token and head
constexpr int kScaleRow = kHeadDim / kGroup;  // 8 scale bytes per token and head
constexpr int kCodePage = kBlockTokens * kCodeRow;    // 8 KiB per (page, head)
constexpr int kScalePage = kBlockTokens * kScaleRow;  // 1 KiB per (page, head)
constexpr int kHeadsPerKv = 8;

// Scale bytes of one (page, head) are stored tile-major: the scale of row r
// (token slot in the page) and 16-channel group g sits at
//   ((g / 2) * 16 + r % 16) * 16 + (r / 16) * 2 + g % 2,
// so the lane that handles rows r % 16 == i and channel slice g / 2 == c in
// every 16-row tile finds all 8 tiles' scale pairs in one 16-byte word.
__host__ __device__ constexpr int scale_offset(int row, int group) {
  return ((group >> 1) * 16 + (row & 15)) * 16 + (row >> 4) * 2 + (group & 1);
}
// byte offset of the 16-byte scale word of lane (slice c, row-in-tile i)
__host__ __device__ constexpr int scale_word_offset(int slice, int row_in_tile) {
  return (slice * 16 + row_in_tile) * 16;
}
// the two scale bytes (groups 2c, 2c+1) of tile j from a lane's scale word
__device__ __forceinline__ uint32_t tile_scales(const uint4& w, int j) {
  const uint32_t d = j < 2 ? w.x : (j < 4 ? w.y : (j < 6 ? w.z : w.w));
  return (j & 1) ? (d >> 16) : (d & 0xFFFFu);
}

// ---------------------------------------------------------------- tables
// E4M3 byte b in 0..126 as an integer count of 2^-11 (every E4M3 value and
// every E2M1 x E4M3 product is a multiple of 2^-10, so midpoints are exact).
constexpr int64_t e4m3_units(int b) {
  return ((b >> 3) & 15) == 0 ? int64_t(b & 7) << 2
                              : int64_t(8 + (b & 7)) << (((b >> 3) & 15) + 1);
}

// Nearest E4M3 byte (0..126) to a non-negative value given as twice its
// count of 2^-11; ties to the even byte; saturates at 448.
constexpr int e4m3_nearest_twice_units(int64_t v2) {
  int best = 0;
  for (int k = 0; k < 126; ++k) {
    const int64_t mid2 = e4m3_units(k) + e4m3_units(k + 1);
    if (v2 > mid2) {
      best = k + 1;
    } else {
      if (v2 == mid2) best = (k % 2 == 0) ? k : k + 1;
      break;
    }
  }
  return best;
}

struct Fp8Lut {
  uint32_t lo[128];  // bytes for magnitudes 0, .5, 1, 1.5
  uint32_t hi[128];  // bytes for magnitudes 2, 3, 4, 6
};

constexpr Fp8Lut make_fp8_lut() {
  Fp8Lut t{};
  constexpr int twice_mag[8] = {0, 1, 2, 3, 4, 6, 8, 12};  // 2 * E2M1 magnitude
  for (int s = 0; s < 128; ++s) {
    uint32_t lo = 0, hi = 0;
    for (int m = 0; m < 8; ++m) {
      // scale byte 0x7F is the E4M3 NaN: its row is NaN (never produced by
      // the quantiser; only reachable through unwritten pool bytes)
      const uint32_t byte =
          s == 127 ? 0x7Fu : uint32_t(e4m3_nearest_twice_units(twice_mag[m] * e4m3_units(s)));
      if (m < 4) lo |= byte << (8 * m);
      else hi |= byte << (8 * (m - 4));
    }
    t.lo[s] = lo;
    t.hi[s] = hi;
  }
  return t;
}

// amax bounds of the scale bytes: b[k] and b[k + 1] are 6 x the midpoints
// of E4M3 byte k with its lower and upper neighbour, exact in fp32 (at most
// 7 significant bits); b[0] = -1 lies below every amax and b[127] = +inf
// above every finite one (byte 126, 448, is the largest finite E4M3).
struct ScaleBounds {
  float b[128];
};

constexpr ScaleBounds make_scale_bounds() {
  ScaleBounds r{};
  r.b[0] = -1.0f;
  for (int k = 0; k < 126; ++k)
    r.b[k + 1] = float(3 * (e4m3_units(k) + e4m3_units(k + 1))) * (1.0f / 2048.0f);
  r.b[127] = __builtin_huge_valf();
  return r;
}

// E4M3 byte 0..126 -> float (exact).
constexpr float e4m3_to_float(int b) { return float(e4m3_units(b)) * (1.0f / 2048.0f); }

// ---------------------------------------------------------------- dequant
// Four FP8 bytes for the even elements (low nibbles) / odd elements (high
// nibbles) of one code dword, given the LUT row (lo, hi) of their scale.
__device__ __forceinline__ uint32_t fp8_even(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  return __builtin_amdgcn_perm(lut_hi, lut_lo, w & 0x07070707u) | ((w << 4) & 0x80808080u);
}
__device__ __forceinline__ uint32_t fp8_odd(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  return __builtin_amdgcn_perm(lut_hi, lut_lo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
}

// 32 consecutive channels of one token row (16 code bytes, two 16-channel
// groups with LUT rows l0 and l1) -> one FP8 MFMA operand (32 bytes). The
// channel order inside each 8-channel run becomes 0,2,4,6,1,3,5,7; the query
// operand is built in the same order (q_operand), and a dot product does
// not depend on it.
__device__ __forceinline__ v8i dequant32(uint4 c, uint2 l0, uint2 l1) {
  v8i r;
  r[0] = (int)fp8_even(c.x, l0.x, l0.y);
  r[1] = (int)fp8_odd(c.x, l0.x, l0.y);
  r[2] = (int)fp8_even(c.y, l0.x, l0.y);
  r[3] = (int)fp8_odd(c.y, l0.x, l0.y);
  r[4] = (int)fp8_even(c.z, l1.x, l1.y);
  r[5] = (int)fp8_odd(c.z, l1.x, l1.y);
  r[6] = (int)fp8_even(c.w, l1.x, l1.y);
  r[7] = (int)fp8_odd(c.w, l1.x, l1.y);
  return r;
}

// 32 consecutive FP8 query bytes -> operand in dequant32's channel order.
__device__ __forceinline__ v8i q_operand(uint4 a, uint4 b) {
  v8i r;
  r[0] = (int)__builtin_amdgcn_perm(a.y, a.x, 0x06040200u);
  r[1] = (int)__builtin_amdgcn_perm(a.y, a.x, 0x07050301u);
  r[2] = (int)__builtin_amdgcn_perm(a.w, a.z, 0x06040200u);
  r[3] = (int)__builtin_amdgcn_perm(a.w, a.z, 0x07050301u);
  r[4] = (int)__builtin_amdgcn_perm(b.y, b.x, 0x06040200u);
  r[5] = (int)__builtin_amdgcn_perm(b.y, b.x, 0x07050301u);
  r[6] = (int)__builtin_amdgcn_perm(b.w, b.z, 0x06040200u);
  r[7] = (int)__builtin_amdgcn_perm(b.w, b.z, 0x07050301u);
  return r;
}

// D(16x16, fp32) = A(16x128, FP8 E4M3) x B(128x16, FP8 E4M3) + C. Lane l
// supplies row l%16 of A and column l%16 of B, 32 bytes each and the same 32
// elements of the reduction dimension: bytes 0-15 are elements 16(l/16) ..
// 16(l/16)+15, bytes 16-31 are 64 + 16(l/16) .. 64 + 16(l/16)+15 (measured
// on gfx950). It receives D rows 4*(l/16) .. 4*(l/16)+3 of column l%16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------- loads
// 16-byte global load with the non-temporal hint: cache data that is streamed
// once (the whole index cache every step, each selected K/V block once) is
// read without displacing reusable lines, which measures ~17% faster on the
// index scan than an ordinary load.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// A buffer descriptor over `bytes` bytes at `base` (gfx9 layout: stride 0,
// default format word). A buffer load past the record count returns zeros
// and reads no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}

constexpr int kLoadNonTemporal = 2;  // buffer-load cache policy: streamed, not kept (nt)

// 16 bytes at lane_off + uniform_off of a descriptor's range, non-temporal.
__device__ __forceinline__ uint4 load_tile16(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int uniform_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, uniform_off, kLoadNonTemporal);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// 4 bytes likewise.
__device__ __forceinline__ uint32_t load_tile4(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int uniform_off) {
  return uint32_t(__builtin_amdgcn_raw_buffer_load_b32(r, lane_off, uniform_off, kLoadNonTemporal));
}

// ---------------------------------------------------------------- waves
// Prefix maximum of an unsigned value inside each row of 16 lanes, with DPP
// row shifts (out-of-row lanes read 0, the identity): lane 15 of a row ends
// with the row's maximum. No LDS round trips, unlike a shuffle butterfly.
// Non-negative floats can use it on their bit patterns.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x111, 0xF, 0xF, true)));  // row_shr:1
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x112, 0xF, 0xF, true)));  // row_shr:2
  v = max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x114, 0xF, 0xF, true)));  // row_shr:4
  return max(v, uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x118, 0xF, 0xF, true)));  // row_shr:8
}
// Maximum of a 64-bit key over the wavefront (xor butterfly), uniform result.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}
// LDS visibility between lanes of one wavefront.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace msa
