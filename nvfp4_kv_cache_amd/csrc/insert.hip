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
// One workgroup per two tokens, 256 threads: eight lanes per 128-channel
// head row (lane g of a row holds channels 16g .. 16g+15), 32 rows per pass
// over the two tokens' rows (152 rows: 5 passes at 95% occupancy). Per
// token, LDS tables fold RMSNorm's weights into RoPE: for each channel c of
// the query heads and of the key heads, A = w_c cos and B = -+ w_p sin
// (partner p = c +- r/2), so an element costs y = inv * (x A + x_p B), with
// inv = 1/sqrt(mean(x^2) + eps) of its row and x_p its partner's raw value.
// The angles pos * theta^(-2i/r) are formed (theta^(-2i/r) as
// exp2(-2i/r * log2 theta)) and reduced modulo 2 pi in fp64, their cosine and
// sine taken in fp32; everything else is fp32:
//   - the row's sum of squares over its eight lanes (xor shuffles);
//   - the partner values by a lane shuffle (lane g with g +- r/32);
//   - K, V, index keys: NVFP4 group encoding (nvfp4_encode_group), 8 code
//     bytes and one scale byte into the token's page row; V is neither
//     normalised nor rotated;
//   - queries: E4M3 (nearest even, clamped to +-448) with the hardware
//     conversion, 16 bytes per lane.
// Without RoPE the B term is not formed, and without normalisation either,
// the inputs reach the encoders unchanged.
#include <cmath>

#include "msa_nvfp4.h"
#include "nvfp4_encode.h"

namespace msa {

__constant__ ScaleThresholds kInsertThr = make_scale_thresholds();

struct InsertArgs {
  const uint16_t* qkv;  // bf16 [T][rows * 128]
  int64_t num_tokens;
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
  double log2_theta;  // log2(theta), from the host's libm in fp64
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

constexpr int kInsertThreads = 256;                      // 4 wavefronts
constexpr int kInsertRowsPerPass = kInsertThreads / 8;   // 32 head rows
constexpr int kInsertTokens = 2;                         // tokens per workgroup
constexpr int kMaxRowsPerToken = 2 * kHeadsPerKv * MSA_MAX_HEADS + 3 * MSA_MAX_HEADS;

__global__ __launch_bounds__(kInsertThreads) void qkv_rope_insert_kernel(const InsertArgs a) {
  __shared__ float thr[128];
  __shared__ float2 csn[kInsertTokens][64];  // cos, sin per angle
  // [token][query, key class][A, B][channel]
  __shared__ __attribute__((aligned(16))) float tab[kInsertTokens][2][2][128];
  __shared__ uint16_t rowinfo[kMaxRowsPerToken];  // kind << 8 | head, per row of a token
  // ids through the builtins: this file is built without IEEE NaN handling,
  // so the device library's id functions would not be inlined but called
  const int tid = int(__builtin_amdgcn_workitem_id_x());
  const int64_t t0 = int64_t(__builtin_amdgcn_workgroup_id_x()) * kInsertTokens;
  const int ntok = int(min(int64_t(kInsertTokens), a.num_tokens - t0));
  const int nrows = ntok * a.rows;  // the workgroup's head rows, token-major
  const int half = a.rotary_dim >> 1;
  const int hq = kHeadsPerKv * a.hkv, hqi = kHeadsPerKv * a.hidx;
  const int g = tid & 7;
  // the tokens' rows are contiguous, so the workgroup's rows are one range;
  // the first pass's loads go out before anything else, so their latency
  // overlaps the table set-up, and each later pass is loaded while the
  // previous one is computed
  const uint16_t* src = a.qkv + t0 * int64_t(a.rows) * kHeadDim;
  auto load_rows = [&](int r0, uint4& u0, uint4& u1) {
    const int r = r0 + (tid >> 3);
    if (r < nrows) {
      const uint4* p = reinterpret_cast<const uint4*>(src + int64_t(r) * kHeadDim + 16 * g);
      u0 = p[0];
      u1 = p[1];
    } else {
      u0 = u1 = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 c0, c1;
  load_rows(0, c0, c1);
  if (tid < 128) thr[tid] = kInsertThr.t[tid];
  const int b1 = hq, b2 = hq + hqi, b3 = b2 + a.hkv, b4 = b3 + a.hkv;
  for (int r = tid; r < a.rows; r += kInsertThreads) {
    // kind: 0 q, 1 q_idx, 2 k, 3 v, 4 k_idx
    const int kind = (r >= b1) + (r >= b2) + (r >= b3) + (r >= b4);
    const int head = r - (kind == 0 ? 0 : kind == 1 ? b1 : kind == 2 ? b2 : kind == 3 ? b3 : b4);
    rowinfo[r] = uint16_t(kind << 8 | head);
  }
  if (tid < kInsertTokens * 64) {
    const int tt = tid >> 6, i = tid & 63;
    if (i < half && tt < ntok) {
      // angle = pos * theta^(-2i/r): the frequency, the product and its reduction modulo
      // 2 pi (two-term Cody-Waite split, fma) in fp64, so long positions
      // keep their accuracy; the cosine and sine of the reduced angle in fp32
      const double inv_freq = exp2(-2.0 * double(i) / double(a.rotary_dim) * a.log2_theta);
      const double ang = double(a.positions[t0 + tt]) * inv_freq;
      constexpr double kTwoPiHi = 6.283185307179586232e+00;   // 2 pi rounded to double
      constexpr double kTwoPiLo = 2.449293598294706414e-16;   // 2 pi - kTwoPiHi
      const double k = rint(ang * (1.0 / kTwoPiHi));
      const float red = float(fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang)));
      csn[tt][i] = make_float2(cosf(red), sinf(red));
    }
  }
  __syncthreads();
#pragma unroll
  for (int tt = 0; tt < kInsertTokens; ++tt) {
    // Per channel of the token's query (class 0) and key (class 1) heads:
    // with weight w (1 without normalisation), y = inv * (x A + x_p B) is
    // RMSNorm then RoPE, A = w_c cos, B = -+ w_p sin for the partner channel
    // p = c +- r/2 of the lower / upper half; A = w_c, B = 0 past r
    const int cls = tid >> 7, c = tid & 127;
    const float* w = cls ? a.k_norm_w : a.q_norm_w;
    float A = w ? w[c] : 1.0f, B = 0.0f;
    if (c < a.rotary_dim) {
      const bool lower = c < half;
      const int ai = lower ? c : c - half, pc = lower ? c + half : c - half;
      const float2 v = csn[tt][ai];
      A *= v.x;
      B = (lower ? -1.0f : 1.0f) * (w ? w[pc] : 1.0f) * v.y;
    }
    tab[tt][cls][0][c] = A;
    tab[tt][cls][1][c] = B;
  }
  __syncthreads();

  const int hg = a.rotary_dim >> 5;  // 16-channel groups in each half (r / 32)
  const int partner = ((tid & 63) & ~7) + (g < hg ? g + hg : g >= 2 * hg ? g : g - hg);

  for (int r0 = 0; r0 < nrows; r0 += kInsertRowsPerPass) {
    const int rr = r0 + (tid >> 3);
    const bool in = rr < nrows;
    const int tt = rr >= a.rows ? 1 : 0;  // kInsertTokens == 2
    const int r = min(rr - tt * a.rows, a.rows - 1);
    const int64_t t = t0 + tt;
    const uint32_t info = rowinfo[r];
    const int kind = int(info >> 8), head = int(info & 0xFFu);
    float x[16];
    {
      const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
    if (r0 + kInsertRowsPerPass < nrows) load_rows(r0 + kInsertRowsPerPass, c0, c1);
    const int cls = kind <= 1 ? 0 : 1;
    const bool qk = kind != 3;
    const bool norm = cls == 0 ? a.q_norm_w != nullptr : a.k_norm_w != nullptr;
    // RMSNorm's scale (the eight lanes of a row share the sum of squares)
    float inv = 1.0f;
    if (a.q_norm_w || a.k_norm_w) {
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(x[i], x[i], ss);
      ss += __shfl_xor(ss, 1, 64);
      ss += __shfl_xor(ss, 2, 64);
      ss += __shfl_xor(ss, 4, 64);
      if (norm) inv = __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + a.eps);
    }
    const float4* A4 = reinterpret_cast<const float4*>(&tab[tt][cls][0][16 * g]);
    if (a.rotary_dim > 0) {
      // every lane shuffles; V lanes keep their values
      float xp[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) xp[i] = __shfl(x[i], partner, 64);
      const float4* B4 = reinterpret_cast<const float4*>(&tab[tt][cls][1][16 * g]);
      if (qk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 av = A4[j], bv = B4[j];
          const float aa[4] = {av.x, av.y, av.z, av.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[4 * j + e] = inv * fmaf(x[4 * j + e], aa[e], xp[4 * j + e] * bb[e]);
        }
      }
    } else if (qk && norm) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 av = A4[j];
        const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * j + e] = inv * (x[4 * j + e] * aa[e]);
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
      const int64_t slot = a.slot_mapping[t];
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
  a.num_tokens = num_tokens;
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
  a.log2_theta = std::log2(double(rope_theta));
  a.q_fp8 = q_fp8;
  a.qi_fp8 = q_idx_fp8;
  hipLaunchKernelGGL(qkv_rope_insert_kernel,
                     dim3(unsigned((num_tokens + kInsertTokens - 1) / kInsertTokens)),
                     dim3(kInsertThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
