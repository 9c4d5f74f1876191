// insert.hip -- msa_qkv_rope_insert: the cache-insertion path after the QKV
// projection, in one launch. The pages describe a fused projection,
// normalisation, RoPE and cache-insertion path that avoids writing the full
// intermediate tensor to HBM and reading it back (MiniMax-M3.1-Flash serving
// summary, section "Reduce both data movement and resource waits"); the
// projection needs model weights and stays outside. Here the projection
// output (bf16) is read once; the normalised, rotated values exist only in
// registers, and what leaves the kernel is the NVFP4 K / V / index-key rows
// in their pages and the FP8 attention and index queries.
//
// One workgroup per token, 256 threads: eight lanes per 128-channel head row
// (lane g of a row holds channels 16g .. 16g+15), 32 rows per pass. The
// token's RoPE cos/sin (at most 64 angles) are evaluated once in fp64 and
// staged in LDS as fp32; everything else is fp32:
//   - RMSNorm: the row's sum of squares over its eight lanes (xor shuffles),
//     x * (1 / sqrt(mean + eps)) * w;
//   - RoPE (rotate-half): channel i < r/2 pairs with i + r/2, i.e. lane g
//     with lane g +- r/32 of the same row (a shuffle per element);
//   - K, V, index keys: NVFP4 group encoding (nvfp4_encode_group), 8 code
//     bytes and one scale byte into the token's page row;
//   - queries: E4M3 (nearest even, clamped to +-448) with the hardware
//     conversion, 16 bytes per lane.
#include <math.h>

#include "msa_nvfp4.h"
#include "nvfp4_tile.h"

namespace msa {

__constant__ ScaleThresholds kInsertThr = make_scale_thresholds();

struct InsertArgs {
  const uint16_t* qkv;  // bf16 [T][rows * 128]
  int rows;             // heads per token row: 8 hkv + 8 hidx + 2 hkv + hidx
  int hkv, hidx;
  const int32_t* positions;
  const int64_t* slot_mapping;
  uint8_t* k_codes;
  uint8_t* k_scales;
  uint8_t* v_codes;
  uint8_t* v_scales;
  int64_t kv_slots;  // pages * 128
  uint8_t* i_codes;
  uint8_t* i_scales;
  int64_t idx_slots;
  const float* q_norm_w;  // [128] or null
  const float* k_norm_w;  // [128] or null
  float eps;
  int rotary_dim;  // 0, 32, 64, 96 or 128
  float theta;
  uint8_t* q_fp8;   // [T][8 hkv][128]
  uint8_t* qi_fp8;  // [T][8 hidx][128]
};

// fp32 -> E4M3 byte: the hardware conversion rounds to nearest even; values
// beyond the largest finite magnitude are clamped to it first (satfinite).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const float m = 448.0f;
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -m), m), fminf(fmaxf(b, -m), m), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -m), m), fminf(fmaxf(d, -m), m), r, true);
  return uint32_t(r);
}

__global__ __launch_bounds__(256) void qkv_rope_insert_kernel(const InsertArgs a) {
  __shared__ float thr[128];
  __shared__ float cs[64], sn[64];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  if (tid < 128) thr[tid] = kInsertThr.t[tid];
  const int half = a.rotary_dim >> 1;
  if (tid < half) {
    // angle = pos * theta^(-2i/r), in fp64 so that long positions keep
    // their accuracy; the rotation itself is fp32
    const double inv = pow(double(a.theta), -2.0 * double(tid) / double(a.rotary_dim));
    const double ang = double(a.positions[t]) * inv;
    cs[tid] = float(cos(ang));
    sn[tid] = float(sin(ang));
  }
  __syncthreads();

  const int hq = kHeadsPerKv * a.hkv, hqi = kHeadsPerKv * a.hidx;
  const int g = tid & 7;
  const int row_lane0 = (tid & 63) & ~7;
  const int64_t slot = a.slot_mapping[t];
  const int rg = a.rotary_dim >> 4;  // rotary groups of 16 channels (r / 16)
  const int hg = rg >> 1;            // groups in each half (r / 32)
  const bool rot = g < rg;
  const int partner = row_lane0 + (g < hg ? g + hg : g - hg);
  const uint16_t* src_t = a.qkv + t * int64_t(a.rows) * kHeadDim;

  for (int r0 = 0; r0 < a.rows; r0 += 32) {
    const int r = r0 + (tid >> 3);
    // kind: 0 q, 1 q_idx, 2 k, 3 v, 4 k_idx (rows past the end: none)
    const bool in = r < a.rows;
    const int kind = r < hq ? 0 : r < hq + hqi ? 1 : r < hq + hqi + a.hkv ? 2
                   : r < hq + hqi + 2 * a.hkv ? 3 : 4;
    const int head = kind == 0 ? r : kind == 1 ? r - hq : kind == 2 ? r - hq - hqi
                   : kind == 3 ? r - hq - hqi - a.hkv : r - hq - hqi - 2 * a.hkv;
    float x[16];
    if (in) {
      const uint4* p = reinterpret_cast<const uint4*>(src_t + int64_t(r) * kHeadDim + 16 * g);
      const uint4 u0 = p[0], u1 = p[1];
      const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.0f;
    }
    // RMSNorm (the eight lanes of a row share the sum; every lane shuffles)
    const float* nw = kind == 0 || kind == 1 ? a.q_norm_w : kind == 3 ? nullptr : a.k_norm_w;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += x[i] * x[i];
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    ss += __shfl_xor(ss, 4, 64);
    if (nw) {
      const float inv = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = x[i] * inv * nw[16 * g + i];
    }
    // RoPE (every lane shuffles; only rotary lanes of rotated kinds use it)
    const bool rotate = rot && kind != 3;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float xp = __shfl(x[i], partner, 64);
      if (rotate) {
        const int c = 16 * g + i;
        if (g < hg) x[i] = x[i] * cs[c] - xp * sn[c];
        else x[i] = x[i] * cs[c - half] + xp * sn[c - half];
      }
    }
    if (!in) continue;
    if (kind <= 1) {
      uint8_t* dst = (kind == 0 ? a.q_fp8 + (t * hq + head) * kHeadDim
                                : a.qi_fp8 + (t * hqi + head) * kHeadDim) + 16 * g;
      *reinterpret_cast<uint4*>(dst) =
          make_uint4(e4m3_pack4(x[0], x[1], x[2], x[3]), e4m3_pack4(x[4], x[5], x[6], x[7]),
                     e4m3_pack4(x[8], x[9], x[10], x[11]), e4m3_pack4(x[12], x[13], x[14], x[15]));
    } else {
      const int64_t nslots = kind == 4 ? a.idx_slots : a.kv_slots;
      if (slot < 0 || slot >= nslots) continue;
      uint8_t* codes = kind == 2 ? a.k_codes : kind == 3 ? a.v_codes : a.i_codes;
      uint8_t* scales = kind == 2 ? a.k_scales : kind == 3 ? a.v_scales : a.i_scales;
      const int nh = kind == 4 ? a.hidx : a.hkv;
      uint32_t packed[2];
      const int sb = nvfp4_encode_group(x, thr, packed);
      const int64_t page_head = (slot / kBlockTokens) * nh + head;
      const int prow = int(slot % kBlockTokens);
      *reinterpret_cast<uint2*>(codes + (page_head * kBlockTokens + prow) * kCodeRow + g * 8) =
          make_uint2(packed[0], packed[1]);
      scales[page_head * kScalePage + scale_offset(prow, g)] = uint8_t(sb);
    }
  }
}

static bool misaligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) != 0; }

static msa_status check_pool(const msa_pool_desc* d) {
  if (!d) return MSA_ERR_INVALID_ARG;
  if (d->head_dim != MSA_HEAD_DIM || d->block_tokens != MSA_BLOCK_TOKENS) return MSA_ERR_UNSUPPORTED;
  if (d->num_heads < 1 || d->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (d->num_pages <= 0 || d->num_pages > (int64_t(1) << 40)) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

}  // namespace msa

extern "C" msa_status msa_qkv_rope_insert(
    const uint16_t* qkv, int64_t num_tokens, const int32_t* positions, const int64_t* slot_mapping,
    const msa_pool_desc* kv, uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
    uint8_t* v_scales, const msa_pool_desc* idx, uint8_t* idx_codes, uint8_t* idx_scales,
    const float* q_norm_w, const float* k_norm_w, float rms_eps, int32_t rotary_dim,
    float rope_theta, uint8_t* q_fp8, uint8_t* q_idx_fp8, void* stream) {
  using namespace msa;
  if (num_tokens < 0) return MSA_ERR_INVALID_ARG;
  msa_status st = check_pool(kv);
  if (st != MSA_OK) return st;
  if ((st = check_pool(idx)) != MSA_OK) return st;
  if (rotary_dim < 0 || rotary_dim > MSA_HEAD_DIM || rotary_dim % 32 != 0) return MSA_ERR_UNSUPPORTED;
  if (rotary_dim > 0 && !(rope_theta > 1.0f && rope_theta < 1e30f)) return MSA_ERR_INVALID_ARG;
  if ((q_norm_w || k_norm_w) && !(rms_eps >= 0.0f && rms_eps < 1e30f)) return MSA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MSA_OK;
  if (num_tokens > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  if (!qkv || !positions || !slot_mapping || !k_codes || !k_scales || !v_codes || !v_scales ||
      !idx_codes || !idx_scales || !q_fp8 || !q_idx_fp8)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(qkv, 15) || misaligned(q_fp8, 15) || misaligned(q_idx_fp8, 15) ||
      misaligned(k_codes, 7) || misaligned(v_codes, 7) || misaligned(idx_codes, 7) ||
      misaligned(positions, 3) || misaligned(slot_mapping, 7) || misaligned(q_norm_w, 3) ||
      misaligned(k_norm_w, 3))
    return MSA_ERR_INVALID_ARG;
  InsertArgs a{};
  a.qkv = qkv;
  a.hkv = kv->num_heads;
  a.hidx = idx->num_heads;
  a.rows = kHeadsPerKv * (a.hkv + a.hidx) + 2 * a.hkv + a.hidx;
  a.positions = positions;
  a.slot_mapping = slot_mapping;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.kv_slots = kv->num_pages * MSA_BLOCK_TOKENS;
  a.i_codes = idx_codes;
  a.i_scales = idx_scales;
  a.idx_slots = idx->num_pages * MSA_BLOCK_TOKENS;
  a.q_norm_w = q_norm_w;
  a.k_norm_w = k_norm_w;
  a.eps = rms_eps;
  a.rotary_dim = rotary_dim;
  a.theta = rope_theta;
  a.q_fp8 = q_fp8;
  a.qi_fp8 = q_idx_fp8;
  hipLaunchKernelGGL(qkv_rope_insert_kernel, dim3(unsigned(num_tokens)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
