// attn_body.h -- one workgroup of the sparse attention (msa_sparse_attn_decode,
// msa_sparse_attn_select_decode and the one-launch decode step): exact GQA
// attention of one query token and KV head over selected 128-token blocks,
// with the NVFP4 K and V pages converted to FP8 through the lookup table
// before the products, and the log-sum-exp merge of split partials.
//
// The pages: main attention runs over the roughly 2,048 keys of the selected
// blocks, exactly (MiniMax-M3.1-Flash serving summary, section "Sparse
// attention still scans an index"); the NVFP4 cache is converted to FP8
// because the query stays FP8 (MiniMax-M3.1-Flash lands in vLLM on day one,
// third paragraph).
#pragma once

#include "msa_nvfp4.h"
#include "nvfp4_tile.h"
#include "topk_select.h"

namespace msa {

struct AttnArgs {
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* v_codes;
  const uint8_t* v_scales;
  int64_t num_pages;
  int num_kv_heads;
  const uint8_t* q;
  int num_q_heads;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  int q_per_seq;
  const int32_t* sel_ids;  // caller's selection [T_q][num_sel], or
  const float* bscore;     // block scores [T_q][max_blocks] to select from
  int32_t* out_ids;        // selection output [T_q][17] (optional, selecting kernel)
  int num_sel;
  int slots_per_wg;    // selected slots per workgroup
  int num_splits;
  float scale_log2;    // softmax_scale * log2(e)
  float* part_o;       // [T_q * Hq][num_splits][128] unnormalised, when num_splits > 1
  float* part_ml;      // [T_q * Hq][num_splits][2]
  uint32_t* split_cnt; // [T_q * KV heads] splits arrived, when num_splits > 1 (zero
                       // between launches: the pair's last split resets it)
  float* out;
};

typedef float v2f __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kAttnWaves = 4;                         // wavefronts per workgroup
constexpr int kVRow = 136;                            // LDS bytes per V row (128 + pad)
// LDS of one wavefront that takes TOK tokens of a block: V rows, then P_hi
// and P_lo as [token][head] FP8
template <int TOK>
struct WaveLds {
  static constexpr int kV = TOK * kVRow;
  static constexpr int kP = TOK * kHeadsPerKv;
  static constexpr int kBytes = kV + 2 * kP;
};
constexpr float kPScaleLog2 = 8.0f;                   // P_hi = FP8(2^8 p)
constexpr float kPLoScale = 16.0f;                    // P_lo = FP8(16 (2^8 p - P_hi))
constexpr int kE8M0One = 0x7F7F7F7F;                  // MFMA operand scale 2^0
constexpr int kE8M0Sixteenth = 0x7B7B7B7B;            // MFMA operand scale 2^-4
constexpr int kFp8Ones = 0x38383838;                  // four FP8 E4M3 1.0

// All-reduce over each row of 16 lanes with DPP (no LDS round trips):
// exchange within quads (xor 1, xor 2), then rotate the row by 4 and by 8,
// which brings in the other three quads.
template <int kCtrl>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_row<kQuadXor1>(v));
  v = fmaxf(v, dpp_row<kQuadXor2>(v));
  v = fmaxf(v, dpp_row<kRowRor4>(v));
  return fmaxf(v, dpp_row<kRowRor8>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_row<kQuadXor1>(v);
  v += dpp_row<kQuadXor2>(v);
  v += dpp_row<kRowRor4>(v);
  return v + dpp_row<kRowRor8>(v);
}

// The scale bytes of a wavefront's NT tiles from the lane's 16-byte scale
// word (tile-major: tile j's two bytes at bytes 2j, 2j+1): the whole word
// for a whole block, one dword (tiles first, first + 1) for a quarter.
template <int NT>
struct TileScaleWords {
  uint32_t d[NT / 2];
};
template <int NT>
__device__ __forceinline__ TileScaleWords<NT> load_tile_scales(const uint8_t* word, int first) {
  TileScaleWords<NT> r;
  if constexpr (NT == 8) {
    const uint4 w = load_stream16(word);
    r.d[0] = w.x;
    r.d[1] = w.y;
    r.d[2] = w.z;
    r.d[3] = w.w;
  } else {
    static_assert(NT == 2, "whole blocks or quarters");
    r.d[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(word + 2 * first));
  }
  return r;
}
template <int NT>
__device__ __forceinline__ uint32_t scale_pair(const TileScaleWords<NT>& w, int j) {
  return (j & 1) ? (w.d[j >> 1] >> 16) : (w.d[j >> 1] & 0xFFFFu);
}

// 32 bytes of an MFMA operand from four transposed 8-byte LDS reads.
__device__ __forceinline__ v8i tr_operand(const uint8_t* p0, const uint8_t* p1, const uint8_t* p2,
                                          const uint8_t* p3) {
  const v2i a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p0));
  const v2i b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p1));
  const v2i c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p2));
  const v2i d = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(p3));
  return v8i{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Dynamic LDS of a workgroup: the wavefronts' V rows and P, then 64 zero bytes.
template <int TOK>
constexpr size_t attn_lds_bytes() {
  return size_t(kAttnWaves) * WaveLds<TOK>::kBytes + 64;
}

// Where a workgroup's blocks come from.
constexpr int kAttnIds = 0;     // the caller's selected ids (lane l: slot l)
constexpr int kAttnSelect = 1;  // selected in the workgroup from the indexer's block scores
constexpr int kAttnEvery = 2;   // block sp itself, selected or not (the one-launch step:
                                // its partial is merged only if the selection takes it);
                                // partials stored at device scope

// TOK: tokens of a block per wavefront. TOK = 128: each wavefront takes
// whole blocks (slots s, s + 4, ... of its workgroup's range) and runs the
// selection itself (no barrier). TOK = 32: the four wavefronts share every
// block of the workgroup's range, wave w taking tokens 32w .. 32w + 31, which
// cuts the serial work per wavefront for launches with few (query token, KV
// head) pairs; wave 0 selects and hands the slots over through LDS.
// SELECT: the kernel selects the blocks itself from the indexer's block
// scores; otherwise the caller's ids are used.

// Device-scope (sc1) accesses to split partials written and read within
// one launch: coherent across the XCDs' L2 caches. Buffer operations over a
// partial array (the host keeps it below 2 GiB), so a lane moves 16 or 8
// bytes at once; 4-byte device-scope stores measured 4x their bytes in
// memory writes.
constexpr int kDeviceScope = 16;  // buffer cache policy: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void store_device_scope(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ void store_device_scope(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(
      __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, v), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ float4 load_device_scope4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
}
__device__ __forceinline__ float2 load_device_scope2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDeviceScope));
}

// Split partials fetched per round of independent loads in the merge.
constexpr int kMergeChunk = 20;

// Log-sum-exp merge of the n partials of one query-head row, this thread's
// channels (4 of them), returned normalised. fetch(k, v, ml) loads partial k
// (k < n; its 4 channels of o and its (m, l)) and returns false for an empty
// one, which counts as (m, l) = (-inf, 0).
template <class Fetch>
__device__ __forceinline__ float4 merge_row(int n, Fetch fetch) {
  const float ninf = -__builtin_huge_valf();
  float M = ninf, den = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < n; s0 += kMergeChunk) {
    float4 v[kMergeChunk];
    float2 ml[kMergeChunk];
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) {
      if (!(s0 + k < n && fetch(s0 + k, v[k], ml[k]))) {
        v[k] = make_float4(0, 0, 0, 0);
        ml[k] = make_float2(ninf, 0.0f);
      }
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) Mc = fmaxf(Mc, ml[k].x);
    if (Mc == ninf) continue;
    const float r = M == ninf ? 0.0f : exp2f(M - Mc);
    den *= r;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] *= r;
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) {
      const float f = ml[k].x == ninf ? 0.0f : exp2f(ml[k].x - Mc);
      den += f * ml[k].y;
      o[0] += f * v[k].x;
      o[1] += f * v[k].y;
      o[2] += f * v[k].z;
      o[3] += f * v[k].w;
    }
    M = Mc;
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  return make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

}  // namespace msa
