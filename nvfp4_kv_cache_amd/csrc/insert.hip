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
// One workgroup per two tokens, 256 threads (4 wavefronts): eight lanes per
// 128-channel head row, 16 channels (two 16-byte loads) per lane. The
// workgroup's rows are taken in kind-major order (all query rows, then
// index-query, key, value and index-key rows), eight rows to a wavefront
// pass, so a pass holds one kind whenever the head counts are multiples of
// eight over the two tokens; each wavefront runs its own passes (wave,
// wave + 4, ...) with the rows of two later passes in flight. Per token,
// LDS tables fold RMSNorm's weights into RoPE: for each channel c of the
// query heads and of the key heads, A = w_c cos and B = -+ w_p sin (partner
// p = c +- r/2), so an element costs y = x' A + x'_p B with x' = x inv,
// inv = 1/sqrt(mean(x^2) + eps) of its row. The angles pos * theta^(-2i/r)
// are formed (theta^(-2i/r) as exp2(-2i/r * log2 theta)) and reduced modulo
// 2 pi in fp64, their cosine and sine taken in fp32; everything else is fp32:
//   - the row's sum of squares: the bf16 pairs' squares by dot2 on the raw
//     words, then over the row's eight lanes by DPP adds;
//   - the partner values: with a full rotation (r = 128) lanes 4-7 of a row
//     hold channel blocks 7, 6, 5, 4, so the partner block (+- 4) is the
//     mirror lane and its value comes by DPP inside the multiply; shorter
//     rotations use a lane shuffle (lane g with g +- r/32);
//   - K, V, index keys: NVFP4 group encoding (nvfp4_encode_group), 8 code
//     bytes and one scale byte into the token's page row; V is neither
//     normalised nor rotated;
//   - queries: E4M3 (nearest even, clamped to +-448) with the hardware
//     conversion, 16 bytes per lane; the clamp is left out when every
//     query weight is small enough that no output can exceed 448.
// Without RoPE the B term is not formed, and without normalisation either,
// the inputs reach the encoders unchanged.
#include <cmath>

#include "msa_nvfp4.h"
#include "nvfp4_encode.h"

namespace msa {

__constant__ ScaleBounds kInsertBnd = make_scale_bounds();

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

// fp32 -> E4M3 bytes: the hardware conversion rounds to nearest even; values
// beyond the largest finite magnitude are clamped to it first (satfinite)
// unless the caller knows that none can be (CLAMP false). The first
// conversion's upper half is overwritten by the second, so its prior
// contents may be anything (here a's bits).
template <bool CLAMP>
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const float m = 448.0f;
  if (CLAMP) {
    a = fminf(fmaxf(a, -m), m);
    b = fminf(fmaxf(b, -m), m);
    c = fminf(fmaxf(c, -m), m);
    d = fminf(fmaxf(d, -m), m);
  }
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return uint32_t(r);
}
template <bool CLAMP>
__device__ __forceinline__ uint4 e4m3_pack16(const float (&x)[16]) {
  return make_uint4(e4m3_pack4<CLAMP>(x[0], x[1], x[2], x[3]),
                    e4m3_pack4<CLAMP>(x[4], x[5], x[6], x[7]),
                    e4m3_pack4<CLAMP>(x[8], x[9], x[10], x[11]),
                    e4m3_pack4<CLAMP>(x[12], x[13], x[14], x[15]));
}

// Weight magnitude below which normalised query heads need no clamp: the
// RMS-normalised row has sum of squares 128 (to a few fp32 ulps), so an
// element pair has norm at most sqrt(128) = 11.32, and the rotation with
// weights up to |w| keeps an output at or below 11.32 |w| (+ rounding):
// 11.32 x 39 = 441.2 < 448.
constexpr float kNoClampWeight = 39.0f;

// a lane's value from another lane of its 8-lane row, folded into the VALU
// op that consumes it (DPP): quad_perm [1,0,3,2] and [2,3,0,1] (lane xor 1,
// xor 2) and row_half_mirror (lane i of each 8 reads lane 7 - i)
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming (nontemporal) stores for the query and code rows: nothing in
// this kernel reads them back, and marking them so measurably shortens the
// launch (the one-byte scale stores, which the cache merges into lines, are
// left as ordinary stores: marking them too was slower).
__device__ __forceinline__ void store_stream(uint8_t* p, uint4 v) {
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store_stream(uint8_t* p, uint32_t lo, uint32_t hi) {
  const u32x2 t = {lo, hi};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ void unpack_bf16(const uint4 (&u)[2], float (&x)[16]) {
  const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

constexpr int kInsertThreads = 256;  // 4 wavefronts
constexpr int kInsertWaves = kInsertThreads / 64;
constexpr int kInsertTokens = 2;     // tokens per workgroup
constexpr int kInsertDepth = 3;      // passes of rows held per wavefront
constexpr int kMaxRowsPerToken = 2 * kHeadsPerKv * MSA_MAX_HEADS + 3 * MSA_MAX_HEADS;

// ROPE: 0 none; 1 rotary_dim 32, 64 or 96 (partner by lane shuffle);
// 2 rotary_dim 128 (partner by DPP row_half_mirror). NORM: a norm weight
// vector is given for the query or the key heads.
template <int ROPE, bool NORM>
// five wavefronts per SIMD (at most 96 VGPRs): the kernel needs both the
// arithmetic and the loads in flight of the extra wavefront
__global__ __launch_bounds__(kInsertThreads) __attribute__((amdgpu_waves_per_eu(5)))
void qkv_rope_insert_kernel(const InsertArgs a) {
  __shared__ float bnd[128];
  __shared__ float2 csn[kInsertTokens][64];  // cos, sin per angle
  // [token][query, key class][A, B][channel]
  __shared__ __attribute__((aligned(16))) float tab[kInsertTokens][2][2][128];
  __shared__ uint32_t vmap[kInsertTokens * kMaxRowsPerToken];
  __shared__ int64_t slot_s[kInsertTokens];
  // ids through the builtins: this file is built without IEEE NaN handling,
  // so the device library's id functions would not be inlined but called
  const int tid = int(__builtin_amdgcn_workitem_id_x());
  const int wave = tid >> 6, lane = tid & 63, rl = lane >> 3, g = lane & 7;
  // the 16-channel block lane g of a row holds: with a full rotation the
  // upper four lanes take blocks 7, 6, 5, 4, so the rotation partner of
  // every lane (block +- 4) is its mirror in the row
  const int blk = ROPE == 2 ? (g < 4 ? g : 11 - g) : g;
  const int64_t t0 = int64_t(__builtin_amdgcn_workgroup_id_x()) * kInsertTokens;
  const int ntok = int(min(int64_t(kInsertTokens), a.num_tokens - t0));
  const int rows = a.rows, hkv = a.hkv, hidx = a.hidx;
  const int nrows = ntok * rows;  // the workgroup's head rows
  const int hq = kHeadsPerKv * hkv, hqi = kHeadsPerKv * hidx;
  const int half = a.rotary_dim >> 1;
  const bool has_qn = a.q_norm_w != nullptr, has_kn = a.k_norm_w != nullptr;
  const float eps = a.eps;

  // The workgroup's rows in kind-major order (queries, index queries, keys,
  // values, index keys; then token, then head), eight to a wavefront pass,
  // so a pass holds one kind wherever the head counts allow. Entry: source
  // row (token * rows + row in the token) | kind << 10 | token << 13 |
  // head << 15 | token * heads of the kind + head << 22.
  const int n0 = ntok * hq, n1 = n0 + ntok * hqi, n2 = n1 + ntok * hkv, n3 = n2 + ntok * hkv;
  auto row_entry = [=](int v) -> uint32_t {
    // (running selects rather than a switch, which would become a table
    // in private memory)
    int kind = 0, start = 0, nh = hq, base = 0;
    if (v >= n0) kind = 1, start = n0, nh = hqi, base = hq;
    if (v >= n1) kind = 2, start = n1, nh = hkv, base = hq + hqi;
    if (v >= n2) kind = 3, start = n2, nh = hkv, base = hq + hqi + hkv;
    if (v >= n3) kind = 4, start = n3, nh = hidx, base = hq + hqi + 2 * hkv;
    const int off = v - start, tt = off / nh, head = off - tt * nh;
    return uint32_t(tt * rows + base + head) | uint32_t(kind) << 10 | uint32_t(tt) << 13 |
           uint32_t(head) << 15 | uint32_t(off) << 22;
  };
  const uint16_t* src = a.qkv + t0 * int64_t(rows) * kHeadDim + 16 * blk;
  auto issue = [=](uint32_t info, uint4 (&u)[2]) {
    const uint4* p = reinterpret_cast<const uint4*>(src + (info & 0x3FFu) * kHeadDim);
    u[0] = p[0];
    u[1] = p[1];
  };
  // The set-up's own global reads go out first (the norm weights of this
  // thread's table channel and its rotation partner, the tokens' positions
  // and slots, the scale bounds), then the first two passes' rows: waiting
  // for the former leaves the rows in flight during the set-up. Later
  // passes are loaded two passes ahead of their use.
  const int cls_t = tid >> 7, c_t = tid & 127;
  const float* w_t = cls_t ? a.k_norm_w : a.q_norm_w;
  const int pc_t = c_t >= a.rotary_dim ? c_t : c_t < half ? c_t + half : c_t - half;
  float wc_t = 1.0f, wp_t = 1.0f;
  if ((ROPE > 0 || NORM) && w_t) {
    wc_t = w_t[c_t];
    wp_t = w_t[pc_t];
  }
  const int tt_a = tid >> 6, i_a = tid & 63;  // angle i of token tt_a
  const bool angle_t = ROPE > 0 && tid < kInsertTokens * 64 && i_a < half && tt_a < ntok;
  const int32_t pos_t = angle_t ? a.positions[t0 + tt_a] : 0;
  const int64_t slot_t = tid < ntok ? a.slot_mapping[t0 + tid] : -1;
  const float bnd_t = tid < 128 ? kInsertBnd.b[tid] : 0.0f;

  uint4 ring[kInsertDepth][2];
  uint32_t info[kInsertDepth];
#pragma unroll
  for (int d = 0; d + 1 < kInsertDepth; ++d) {
    info[d] = row_entry(min((wave + d * kInsertWaves) * 8 + rl, nrows - 1));
    issue(info[d], ring[d]);
  }

  for (int v = tid; v < nrows; v += kInsertThreads) vmap[v] = row_entry(v);
  if (tid < 128) bnd[tid] = bnd_t;
  if (tid < kInsertTokens) slot_s[tid] = slot_t;
  if (angle_t) {
    // angle = pos * theta^(-2i/r): the frequency, the product and its reduction modulo
    // 2 pi (two-term Cody-Waite split, fma) in fp64, so long positions
    // keep their accuracy; the cosine and sine of the reduced angle in fp32
    const double inv_freq = exp2(-2.0 * double(i_a) / double(a.rotary_dim) * a.log2_theta);
    const double ang = double(pos_t) * inv_freq;
    constexpr double kTwoPiHi = 6.283185307179586232e+00;   // 2 pi rounded to double
    constexpr double kTwoPiLo = 2.449293598294706414e-16;   // 2 pi - kTwoPiHi
    const double k = rint(ang * (1.0 / kTwoPiHi));
    const float red = float(fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang)));
    csn[tt_a][i_a] = make_float2(cosf(red), sinf(red));
  }
  if (ROPE > 0 || NORM) {
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < kInsertTokens; ++tt) {
      // Per channel of the token's query (class 0) and key (class 1) heads:
      // with weight w (1 without normalisation), y = x' A + x'_p B is RoPE
      // of the normalised x' = x inv, A = w_c cos, B = -+ w_p sin for the
      // partner channel p = c +- r/2 of the lower / upper half; A = w_c,
      // B = 0 past r
      float A = wc_t, B = 0.0f;
      if (c_t < a.rotary_dim) {
        const bool lower = c_t < half;
        const float2 v = csn[tt][lower ? c_t : c_t - half];
        A *= v.x;
        B = (lower ? -1.0f : 1.0f) * wp_t * v.y;
      }
      tab[tt][cls_t][0][c_t] = A;
      tab[tt][cls_t][1][c_t] = B;
    }
  }
  // the query heads need the FP8 clamp unless they are normalised with
  // weights all below kNoClampWeight
  const bool clamp_q =
      __syncthreads_or(cls_t == 0 && !(has_qn && fabsf(wc_t) <= kNoClampWeight)) != 0;

  const int hg = a.rotary_dim >> 5;  // 16-channel blocks in each half (r / 32)
  const int partner = (lane & ~7) + (g < hg ? g + hg : g >= 2 * hg ? g : g - hg);
  uint8_t* const qdst = a.q_fp8 + (t0 * hq) * kHeadDim + 16 * blk;
  uint8_t* const qidst = a.qi_fp8 + (t0 * hqi) * kHeadDim + 16 * blk;
  uint8_t* const codes_of[3] = {a.k_codes, a.v_codes, a.i_codes};
  uint8_t* const scales_of[3] = {a.k_scales, a.v_scales, a.i_scales};
  const int64_t kv_slots = a.kv_slots, idx_slots = a.idx_slots;

  auto process = [&](int wp, const uint4 (&u)[2], uint32_t info) {
    const int v = wp * 8 + rl;
    const int kind = int((info >> 10) & 7u), tt = int((info >> 13) & 3u);
    const int head = int((info >> 15) & 0x7Fu), orow = int(info >> 22);
    float x[16];
    unpack_bf16(u, x);
    if (ROPE > 0 || NORM) {
      // V rows are neither normalised nor rotated: lanes of V rows restore
      // their inputs after the transform
      const bool isv = kind == 3;
      const uint64_t vlanes = __ballot(isv);
      const int cls = kind <= 1 ? 0 : 1;
      if (NORM) {
        // RMSNorm's scale: the eight lanes of a row share the sum of squares
        float ss = 0.0f;
        {
          const uint32_t w[8] = {u[0].x, u[0].y, u[0].z, u[0].w, u[1].x, u[1].y, u[1].z, u[1].w};
#pragma unroll
          for (int i = 0; i < 8; ++i) {  // the two bf16 squares of a word, exact, added in fp32
            const bf16x2 h = __builtin_bit_cast(bf16x2, w[i]);
            ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
          }
        }
        ss += dpp<kDppXor1>(ss);
        ss += dpp<kDppXor2>(ss);
        ss += dpp<kDppHalfMirror>(ss);
        const bool norm = !isv && (cls == 0 ? has_qn : has_kn);
        const float inv = norm ? __builtin_amdgcn_rsqf(ss * (1.0f / kHeadDim) + eps) : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] *= inv;
      }
      const float4* A4 = reinterpret_cast<const float4*>(&tab[tt][cls][0][16 * blk]);
      const float4* B4 = reinterpret_cast<const float4*>(&tab[tt][cls][1][16 * blk]);
      if (ROPE == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 av = A4[j], bv = B4[j];
          const float aa[4] = {av.x, av.y, av.z, av.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            x[4 * j + e] = fmaf(x[4 * j + e], aa[e], dpp<kDppHalfMirror>(x[4 * j + e]) * bb[e]);
        }
      } else if (ROPE == 1) {
        float xp[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          xp[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(partner << 2, __float_as_int(x[i])));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 av = A4[j], bv = B4[j];
          const float aa[4] = {av.x, av.y, av.z, av.w}, bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * j + e] = fmaf(x[4 * j + e], aa[e], xp[4 * j + e] * bb[e]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 av = A4[j];
          const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * j + e] *= aa[e];
        }
      }
      if (vlanes != 0) {
        float x0[16];
        unpack_bf16(u, x0);
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = isv ? x0[i] : x[i];
      }
    }
    if (v >= nrows) return;
    if (kind <= 1) {
      uint8_t* dst = (kind == 0 ? qdst : qidst) + orow * kHeadDim;
      store_stream(dst, clamp_q ? e4m3_pack16<true>(x) : e4m3_pack16<false>(x));
    } else {
      const int64_t slot = slot_s[tt];
      const int64_t nslots = kind == 4 ? idx_slots : kv_slots;
      if (slot < 0 || slot >= nslots) return;
      uint8_t* codes = kind == 2 ? codes_of[0] : kind == 3 ? codes_of[1] : codes_of[2];
      uint8_t* scales = kind == 2 ? scales_of[0] : kind == 3 ? scales_of[1] : scales_of[2];
      const int nh = kind == 4 ? hidx : hkv;
      uint32_t packed[2];
      const int sb = nvfp4_encode_group(x, bnd, packed);
      const int64_t page_head = (slot / kBlockTokens) * nh + head;
      const int prow = int(slot % kBlockTokens);
      store_stream(codes + (page_head * kBlockTokens + prow) * kCodeRow + blk * 8, packed[0],
                   packed[1]);
      scales[page_head * kScalePage + scale_offset(prow, blk)] = uint8_t(sb);
    }
  };

  // wavefront passes wave, wave + 4, ...: kInsertDepth per iteration in
  // rotating register sets, each loaded kInsertDepth - 1 passes ahead. The
  // loads are issued unconditionally (past the last pass they re-read the
  // last row, a cache hit), so the wait before each pass counts exactly the
  // loads issued after its own.
  const int npass = (nrows + 7) >> 3;
  for (int wp = wave; wp < npass; wp += kInsertDepth * kInsertWaves) {
#pragma unroll
    for (int d = 0; d < kInsertDepth; ++d) {
      constexpr int kAhead = kInsertDepth - 1;
      const int nd = (d + kAhead) % kInsertDepth;
      info[nd] = vmap[min((wp + (d + kAhead) * kInsertWaves) * 8 + rl, nrows - 1)];
      issue(info[nd], ring[nd]);
      if (d == 0 || wp + d * kInsertWaves < npass) process(wp + d * kInsertWaves, ring[d], info[d]);
    }
  }
}

template <int ROPE, bool NORM>
static void launch_insert(const InsertArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((qkv_rope_insert_kernel<ROPE, NORM>),
                     dim3(unsigned((a.num_tokens + kInsertTokens - 1) / kInsertTokens)),
                     dim3(kInsertThreads), 0, stream, a);
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
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool norm = q_norm_w || k_norm_w;
  if (rotary_dim == 0) {
    if (norm) launch_insert<0, true>(a, hs);
    else launch_insert<0, false>(a, hs);
  } else if (rotary_dim == MSA_HEAD_DIM) {
    if (norm) launch_insert<2, true>(a, hs);
    else launch_insert<2, false>(a, hs);
  } else {
    if (norm) launch_insert<1, true>(a, hs);
    else launch_insert<1, false>(a, hs);
  }
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
