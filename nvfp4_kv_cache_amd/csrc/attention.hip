// attention.hip -- msa_sparse_attn_decode and msa_sparse_attn_select_decode:
// exact GQA attention of each query token over the visible tokens of its
// selected blocks, with the NVFP4 K and V pages converted to FP8 through the
// lookup table before the products; the second entry point first selects the
// blocks itself from the indexer's block scores (topk_select.h).
//
// The pages: main attention runs over the roughly 2,048 keys of the selected
// blocks, exactly (MiniMax-M3.1-Flash serving summary, section "Sparse
// attention still scans an index"); the NVFP4 cache is converted to FP8
// because the query stays FP8 (MiniMax-M3.1-Flash lands in vLLM on day one,
// third paragraph).
//
// Grid (splits, KV heads, query tokens), 4 wavefronts per workgroup. Split s
// covers selected slots [s*4R, (s+1)*4R); wave w takes slots s*4R + w + 4k,
// k < R, each one 128-token block, keeping its own online-softmax state; the
// waves merge through LDS, and with several splits a second kernel merges
// the splits' (m, l, o) by log-sum-exp. Per block a wave:
//   1. dequantises the 8 K tiles into FP8 MFMA operands and computes
//      S = Q K^T with v_mfma_f32_16x16x128_f8f6f4 (A = the 8 query heads of
//      this KV head, rows 8..15 zero; B = 16 tokens x 128 channels);
//   2. dequantises V into LDS as FP8, one 136-byte row per token, channels
//      in the dequantiser's order (the output index undoes it);
//   3. runs the softmax in base 2 in fp32, scales P by 2^8 and splits it into
//      two FP8 terms, P_hi = FP8(256 p) and P_lo = FP8(16 (256 p - P_hi)), so
//      P_hi + P_lo / 16 carries about 8 significant bits;
//   4. computes O += P_hi V + 2^-4 P_lo V with the same MFMA (the second with
//      its E8M0 operand scale set to 2^-4): all operands are read
//      transposed from LDS with ds_read_b64_tr_b8 (within each 16-lane group,
//      lane i receives byte i%8 of the 8-byte segments addressed by lanes
//      i/8, i/8 + 2, ..., i/8 + 14), so lane i ends with 8 consecutive tokens
//      of one head (P) or one channel (V). The softmax denominator is the
//      same product against FP8 ones, so it sums exactly the terms the
//      numerator uses.
#include "msa_nvfp4.h"
#include "nvfp4_tile.h"
#include "topk_select.h"

namespace msa {

__constant__ Fp8Lut kAttnLut = make_fp8_lut();

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
constexpr float kPScale = 256.0f;                     // P_hi = FP8(256 p)
constexpr float kPLoScale = 16.0f;                    // P_lo = FP8(16 (256 p - P_hi))
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

// TOK: tokens of a block per wavefront. TOK = 128: each wavefront takes
// whole blocks (slots s, s + 4, ... of its workgroup's range) and runs the
// selection itself (no barrier). TOK = 32: the four wavefronts share every
// block of the workgroup's range, wave w taking tokens 32w .. 32w + 31, which
// cuts the serial work per wavefront for launches with few (query token, KV
// head) pairs; wave 0 selects and hands the slots over through LDS.
// SELECT: the kernel selects the blocks itself from the indexer's block
// scores; otherwise the caller's ids are used.
template <int TOK, bool SELECT>
__global__ __launch_bounds__(64 * kAttnWaves)
__attribute__((amdgpu_waves_per_eu(TOK < kBlockTokens ? 3 : 1))) void sparse_attn_kernel(const AttnArgs a) {
  constexpr int W = kAttnWaves;
  static_assert(W == 4, "the workgroup merge maps 256 threads onto 8 heads x 32 channel quads");
  constexpr bool kShared = TOK < kBlockTokens;  // the waves share each block
  static_assert(TOK == kBlockTokens || TOK * W == kBlockTokens, "a block is one wave's or all four's");
  constexpr int NT = TOK / 16;  // 16-token tiles per wavefront
  using WL = WaveLds<TOK>;
  static_assert(sizeof(SelectScratch) <= size_t(kShared ? W : 1) * WL::kBytes,
                "the selection's scratch lives in the V rows");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // W x (V rows, P) + zeros
  __shared__ uint2 lut[128];
  __shared__ int slot_blk[kShared ? 64 : 1], slot_page[kShared ? 64 : 1];

  const int sp = blockIdx.x, kh = blockIdx.y, qt = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int slice = lane >> 4;  // 32-channel slice (QK) / 32-token group (PV)
  const int li = lane & 15;     // row of A / column of B inside a 16-lane group
  const int Q = a.q_per_seq;
  const int b = qt / Q, qi = qt - b * Q;
  const int Hq = a.num_q_heads;
  const bool selector = !kShared || wave_u == 0;  // this wavefront runs the selection
  uint8_t* vrows = smem + wave * WL::kBytes;
  uint8_t* prows = vrows + WL::kV;         // P_hi [token][head]
  uint8_t* plows = prows + WL::kP;         // P_lo [token][head]
  const uint8_t* zeros = smem + W * WL::kBytes;

  // Loads in flight first, oldest first: the query operand (unconditional,
  // rows 8..15 masked afterwards), then this query token's block scores or
  // the caller's ids (lane l: slot l). Load counters retire in order, so a
  // load issued late would later make its consumer wait for every load
  // issued before it.
  const uint4* qp = reinterpret_cast<const uint4*>(
      a.q + (int64_t(qt) * Hq + kh * kHeadsPerKv + (li & (kHeadsPerKv - 1))) * kHeadDim +
      slice * 32);
  uint4 qa = qp[0], qb = qp[1];
  float x0[kSelPerLane];
  int sel = -1;
  if constexpr (SELECT) {
    if (selector) load_score_chunk(a.bscore + int64_t(qt) * a.max_blocks, a.max_blocks, 0, lane, x0);
  } else {
    if (lane < a.num_sel) sel = a.sel_ids[int64_t(qt) * a.num_sel + lane];
  }
  const int L = a.seq_lens[b];
  const bool seq_ok = L >= Q && L <= a.max_blocks * kBlockTokens;
  const int pos = L - Q + qi;

  for (int i = tid; i < 128; i += 64 * W) lut[i] = make_uint2(kAttnLut.lo[i], kAttnLut.hi[i]);
  if (tid < 16) reinterpret_cast<uint32_t*>(smem + W * WL::kBytes)[tid] = 0u;
  // query operand: rows 0..7 = the 8 query heads of this KV head. Consuming
  // the loads here (before anything waits for the later ones) keeps the
  // compiler from sinking them past the selection.
  asm volatile("" : "+v"(qa.x), "+v"(qa.y), "+v"(qa.z), "+v"(qa.w), "+v"(qb.x), "+v"(qb.y),
               "+v"(qb.z), "+v"(qb.w));
  v8i qop = q_operand(qa, qb);
  if (li >= kHeadsPerKv) qop = v8i{0, 0, 0, 0, 0, 0, 0, 0};

  // lane l: block of selected slot l and its physical page (-1: skip). Every
  // wavefront runs the same selection (no barrier, scratch in its own LDS).
  int pg = -1;
  if constexpr (SELECT) {
    if (selector) {
      if (seq_ok) {
        float score;
        int page;
        sel = select_blocks(a.bscore + int64_t(qt) * a.max_blocks, a.max_blocks,
                            pos / kBlockTokens + 1, x0, *reinterpret_cast<SelectScratch*>(vrows),
                            lane, &score, a.block_table + int64_t(b) * a.max_blocks, &page);
        pg = (sel >= 0 && page >= 0 && page < a.num_pages) ? page : -1;
      }
      if (a.out_ids && sp == 0 && kh == 0 && wave_u == 0 && lane <= kTopK)
        a.out_ids[int64_t(qt) * (kTopK + 1) + lane] = sel;
      if (kShared) {
        slot_blk[lane] = sel;
        slot_page[lane] = pg;
      }
    }
  } else {
    if (seq_ok && sel >= 0 && sel < a.max_blocks && sel * kBlockTokens <= pos) {
      const int p = a.block_table[int64_t(b) * a.max_blocks + sel];
      pg = (p >= 0 && p < a.num_pages) ? p : -1;
    }
  }
  // online-softmax state of heads 4*slice + v (meaningful in lanes 0..31)
  const float ninf = -__builtin_huge_valf();
  float m_run[4] = {ninf, ninf, ninf, ninf};
  float l_run[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  v4f o[8];  // rows = heads 4*slice + v, column = channel 16*n + li
#pragma unroll
  for (int n = 0; n < 8; ++n) o[n] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();
  if (SELECT && kShared && !selector) {
    sel = slot_blk[lane];
    pg = slot_page[lane];
  }

  const int64_t page_codes = int64_t(a.num_kv_heads) * kCodePage;
  const int64_t page_scales = int64_t(a.num_kv_heads) * kScalePage;
  const int lane_code = li * kCodeRow + slice * 16;
  const int lane_scale = scale_word_offset(slice, li);
  // transposed-read addresses: segment of lane i = row (i / 2) of an 8-row
  // group, left or right 8 bytes (V) / real or zero segment (P)
  const int seg_row = li >> 1, seg_half = li & 1;

  const int s_begin = sp * a.slots_per_wg;
  const int s_end = min(a.num_sel, s_begin + a.slots_per_wg);
  const int t_wave = kShared ? TOK * wave_u : 0;  // this wavefront's first token of a block
  bool fresh = true;  // no block accumulated yet: o is zero and needs no rescale
  for (int si = s_begin + (kShared ? 0 : wave_u); si < s_end; si += (kShared ? 1 : W)) {
    const int page = __builtin_amdgcn_readlane(pg, si);
    if (page < 0) continue;  // uniform over the wavefront
    const int blk = __builtin_amdgcn_readlane(sel, si);
    // visible tokens of this wavefront's part of the block
    const int nvis = min(TOK, pos + 1 - blk * kBlockTokens - t_wave);
    if (nvis <= 0) continue;  // uniform
    const int64_t hc = int64_t(page) * page_codes + int64_t(kh) * kCodePage + lane_code +
                       int64_t(t_wave) * kCodeRow;
    const int64_t hs = int64_t(page) * page_scales + int64_t(kh) * kScalePage + lane_scale;
    uint4 kc[NT], vc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) kc[j] = load_stream16(a.k_codes + hc + j * 16 * kCodeRow);
    const TileScaleWords<NT> ksw = load_tile_scales<NT>(a.k_scales + hs, t_wave / 16);
#pragma unroll
    for (int j = 0; j < NT; ++j) vc[j] = load_stream16(a.v_codes + hc + j * 16 * kCodeRow);
    const TileScaleWords<NT> vsw = load_tile_scales<NT>(a.v_scales + hs, t_wave / 16);
    // 1. logits of 16 tokens per tile: lane holds heads 4*slice+v, token
    //    t_wave + 16j + li
    const bool part = nvis < TOK;  // this part of the block is only partly visible
    float z[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t ks = scale_pair(ksw, j);
      const v8i kop = dequant32(kc[j], lut[ks & 0x7F], lut[(ks >> 8) & 0x7F]);
      const v4f c = mfma_fp8_16x16x128(qop, kop, v4f{0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
      for (int v = 0; v < 4; ++v) z[j][v] = c[v] * a.scale_log2;
    }
    if (part) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) z[j][v] = 16 * j + li < nvis ? z[j][v] : ninf;
    }
    // 2. V rows into LDS in the dequantiser's channel order (0,2,4,6,1,3,5,7
    //    in every run of 8; the output index undoes it); invisible tokens -> 0
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t vsc = scale_pair(vsw, j);
      v8i vop = dequant32(vc[j], lut[vsc & 0x7F], lut[(vsc >> 8) & 0x7F]);
      if (part && 16 * j + li >= nvis) vop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      uint8_t* dst = vrows + (16 * j + li) * kVRow + slice * 32;
      *reinterpret_cast<uint2*>(dst) = make_uint2(uint32_t(vop[0]), uint32_t(vop[1]));
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(uint32_t(vop[2]), uint32_t(vop[3]));
      *reinterpret_cast<uint2*>(dst + 16) = make_uint2(uint32_t(vop[4]), uint32_t(vop[5]));
      *reinterpret_cast<uint2*>(dst + 24) = make_uint2(uint32_t(vop[6]), uint32_t(vop[7]));
    }
    // 3. softmax: block max per head, rescale, P = FP8(256 * 2^(z - m)) as
    //    two FP8 terms (exp2 of -inf is 0, so invisible tokens drop out)
    float alpha[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mb = z[0][v];
#pragma unroll
      for (int j = 1; j < NT; ++j) mb = fmaxf(mb, z[j][v]);
      const float m_new = fmaxf(m_run[v], row16_max(mb));
      alpha[v] = __builtin_amdgcn_exp2f(m_run[v] - m_new);
      m_run[v] = m_new;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(z[j][v] - m_run[v]) * kPScale;
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
      const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
      const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32((p[0] - h01.x) * kPLoScale,
                                               (p[1] - h01.y) * kPLoScale, 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32((p[2] - h23.x) * kPLoScale,
                                           (p[3] - h23.y) * kPLoScale, lo, true);
      if (lane < 32) {
        const int off = (16 * j + li) * kHeadsPerKv + 4 * slice;
        *reinterpret_cast<int*>(prows + off) = hi;
        *reinterpret_cast<int*>(plows + off) = lo;
      }
    }
    if (!fresh) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n][v] *= alpha[v];
    }
    wave_lds_sync();
    // 4. O += P_hi V + 2^-4 P_lo V. A: lane li < 8 -> head li, tokens
    //    32*slice + 8r .. +7; lanes 8..15 read the zero segment (rows 8..15
    //    of A are zero). The softmax denominator is the same product with a
    //    column of FP8 ones, so it sums exactly the rounded terms of P.
    const v8i ones = v8i{kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones,
                         kFp8Ones, kFp8Ones, kFp8Ones, kFp8Ones};
    if constexpr (kShared) {
      // 32 tokens, one MFMA per 16 channels for both terms. The 16x16x128
      // product takes bytes 0-15 of lane group g as K elements 16g .. 16g+15
      // and bytes 16-31 as 64 + 16g .. 64 + 16g + 15, and the E8M0 scale of
      // lane group c applies to K elements 32c .. 32c + 31 (both measured).
      // Lane groups 0 and 1 carry tokens 16g .. 16g + 15: P_hi in their low
      // halves (K block 0, scale 1), P_lo in their high halves (K block 2,
      // scale 2^-4 from lane group 2); V repeats the same tokens in both
      // halves; lane groups 2 and 3 are zero.
      const bool live = slice < 2;
      const int tok = 16 * slice + seg_row;  // token of this lane's segment (reads 0 and 2)
      const uint8_t* ph = (live && !seg_half) ? prows + tok * kHeadsPerKv : zeros;
      const uint8_t* pl = (live && !seg_half) ? plows + tok * kHeadsPerKv : zeros;
      const int pstep = (live && !seg_half) ? 8 * kHeadsPerKv : 0;
      const v8i pop = tr_operand(ph, ph + pstep, pl, pl + pstep);
      const int pscale = slice == 2 ? kE8M0Sixteenth : kE8M0One;
      const v4f lb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          pop, ones, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, pscale, 0, kE8M0One);
      const uint8_t* vb = live ? vrows + tok * kVRow + 8 * seg_half : zeros;
      const int vstep = live ? 8 * kVRow : 0;
      const int nstep = live ? 16 : 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint8_t* vp = vb + nstep * n;
        const v8i vop = tr_operand(vp, vp + vstep, vp, vp + vstep);
        o[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pop, vop, o[n], 0, 0, 0, pscale, 0,
                                                                 kE8M0One);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) l_run[v] = l_run[v] * alpha[v] + lb[v];
    } else {
      const int t0 = 32 * slice;
      const int poff = (t0 + seg_row) * kHeadsPerKv;
      const uint8_t* ph = seg_half ? zeros : prows + poff;
      const uint8_t* pl = seg_half ? zeros : plows + poff;
      const int pstep = seg_half ? 0 : 8 * kHeadsPerKv;
      const v8i pop_hi = tr_operand(ph, ph + pstep, ph + 2 * pstep, ph + 3 * pstep);
      const v8i pop_lo = tr_operand(pl, pl + pstep, pl + 2 * pstep, pl + 3 * pstep);
      v4f lb = mfma_fp8_16x16x128(pop_hi, ones, v4f{0.0f, 0.0f, 0.0f, 0.0f});
      lb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pop_lo, ones, lb, 0, 0, 0,
                                                           kE8M0Sixteenth, 0, kE8M0One);
      const uint8_t* vb = vrows + (t0 + seg_row) * kVRow + 8 * seg_half;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint8_t* vp = vb + 16 * n;
        const v8i vop = tr_operand(vp, vp + 8 * kVRow, vp + 16 * kVRow, vp + 24 * kVRow);
        o[n] = mfma_fp8_16x16x128(pop_hi, vop, o[n]);
        o[n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pop_lo, vop, o[n], 0, 0, 0,
                                                                 kE8M0Sixteenth, 0, kE8M0One);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) l_run[v] = l_run[v] * alpha[v] + lb[v];
    }
    fresh = false;
    wave_lds_sync();
  }

  // merge the waves' partial results through LDS (reusing the V rows)
  __syncthreads();
  float* mo = reinterpret_cast<float*>(smem);                  // [W][8 heads][128]
  float* mml = mo + W * kHeadsPerKv * kHeadDim;                // [W][8 heads][2]
  // o[n] column li holds V byte 16 n + li of the rows, i.e. channel
  // 16 n + (li & 8) + {0, 2, 4, 6, 1, 3, 5, 7}[li & 7]
  const int chan = (li & 8) + ((li & 7) < 4 ? 2 * (li & 7) : 2 * (li & 7) - 7);
  if (lane < 32) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int h = 4 * slice + v;
#pragma unroll
      for (int n = 0; n < 8; ++n) mo[(wave * kHeadsPerKv + h) * kHeadDim + 16 * n + chan] = o[n][v];
      if (li == 0) {
        mml[(wave * kHeadsPerKv + h) * 2] = m_run[v];
        mml[(wave * kHeadsPerKv + h) * 2 + 1] = l_run[v];
      }
    }
  }
  __syncthreads();
  // thread: head h, channels 4 c .. 4 c + 3
  const int64_t row = int64_t(qt) * Hq + kh * kHeadsPerKv;
  const int h = tid >> 5, d0 = (tid & 31) * 4;
  float M = ninf;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, mml[(w * kHeadsPerKv + h) * 2]);
  float4 num = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  float den = 0.0f;
  if (M != ninf) {
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = mml[(w * kHeadsPerKv + h) * 2];
      const float f = mw == ninf ? 0.0f : exp2f(mw - M);
      den += f * mml[(w * kHeadsPerKv + h) * 2 + 1];
      const float4 ov = *reinterpret_cast<const float4*>(&mo[(w * kHeadsPerKv + h) * kHeadDim + d0]);
      num.x += f * ov.x;
      num.y += f * ov.y;
      num.z += f * ov.z;
      num.w += f * ov.w;
    }
  }
  if (a.num_splits == 1) {
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    *reinterpret_cast<float4*>(&a.out[(row + h) * kHeadDim + d0]) =
        make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
  } else {
    *reinterpret_cast<float4*>(&a.part_o[((row + h) * a.num_splits + sp) * kHeadDim + d0]) = num;
    if (d0 == 0)
      *reinterpret_cast<float2*>(&a.part_ml[((row + h) * a.num_splits + sp) * 2]) = make_float2(M, den);
  }
}

// Merge kernel: one workgroup per (query token, KV head); thread (h, 4 ch)
// combines the splits' (m, l, o) by log-sum-exp. Up to kMergeChunk splits
// are fetched per round of independent loads.
constexpr int kMergeChunk = 20;

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    int num_splits, float* __restrict__ out) {
  const int tid = threadIdx.x;
  const int64_t row = int64_t(blockIdx.x) * kHeadsPerKv + (tid >> 5);  // query head row
  const int pd = (tid & 31) * 4;
  const float* po = part_o + row * num_splits * kHeadDim + pd;
  const float* pm = part_ml + row * num_splits * 2;
  const float ninf = -__builtin_huge_valf();
  float M = ninf, den = 0.0f, o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < num_splits; s0 += kMergeChunk) {
    float4 v[kMergeChunk];
    float2 ml[kMergeChunk];
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) {
      const bool in = s0 + k < num_splits;
      v[k] = in ? *reinterpret_cast<const float4*>(po + (s0 + k) * kHeadDim) : make_float4(0, 0, 0, 0);
      ml[k] = in ? *reinterpret_cast<const float2*>(pm + (s0 + k) * 2) : make_float2(ninf, 0.0f);
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
  *reinterpret_cast<float4*>(out + row * kHeadDim + pd) =
      make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool misaligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) != 0; }

// Launch plan for `pairs` (query token, KV head) pairs and num_sel slots.
// Few pairs (pairs * num_sel <= kSharedMaxWgs): one workgroup per selected
// block, its four wavefronts sharing the block (32 tokens each), so the
// serial work per wavefront is a quarter block. Measured against whole
// blocks per wavefront at 17 slots: 2.3 us faster per step at 4 pairs, 1.5 us
// at 16, 0.4 us slower at 32 (more workgroups than the chip runs evenly).
// Otherwise whole blocks per wavefront: one block per wave while that keeps
// the workgroup count under ~1024, else R blocks per wave.
constexpr int64_t kSharedMaxWgs = 384;
struct AttnPlan {
  int tok;           // tokens of a block per wavefront: 32 or 128
  int slots_per_wg;  // selected slots per workgroup
  int splits;        // workgroups per pair
};
inline AttnPlan attn_plan(int64_t pairs, int num_sel) {
  if (pairs * num_sel <= kSharedMaxWgs) return AttnPlan{kBlockTokens / kAttnWaves, 1, num_sel};
  int R = 1;
  while (R < num_sel && pairs * ((num_sel + kAttnWaves * R - 1) / (kAttnWaves * R)) > 1024) ++R;
  return AttnPlan{kBlockTokens, kAttnWaves * R, (num_sel + kAttnWaves * R - 1) / (kAttnWaves * R)};
}

template <int TOK>
constexpr size_t attn_lds_bytes() {
  return size_t(kAttnWaves) * WaveLds<TOK>::kBytes + 64;
}

}  // namespace msa

extern "C" size_t msa_attn_workspace_bytes(int32_t num_seqs, int32_t q_per_seq,
                                           int32_t num_q_heads, int32_t num_sel) {
  if (num_seqs <= 0 || q_per_seq <= 0 || num_q_heads <= 0 || num_sel <= 0) return 0;
  // the split partials of the launch plan for these shapes
  const int64_t kv_heads = (num_q_heads + MSA_HEADS_PER_KV - 1) / MSA_HEADS_PER_KV;
  const msa::AttnPlan plan = msa::attn_plan(int64_t(num_seqs) * q_per_seq * kv_heads, num_sel);
  if (plan.splits <= 1) return 0;
  const size_t rows = size_t(num_seqs) * q_per_seq * num_q_heads;
  const size_t splits = size_t(plan.splits);
  return msa::align256(rows * splits * MSA_HEAD_DIM * 4) + msa::align256(rows * splits * 2 * 4);
}

namespace msa {

// Host checks shared by both attention entry points.
static msa_status check_attn(const msa_pool_desc* kv, const uint8_t* k_codes,
                             const uint8_t* k_scales, const uint8_t* v_codes,
                             const uint8_t* v_scales, const uint8_t* q_fp8, int32_t num_q_heads,
                             const int32_t* block_table, int32_t max_blocks,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                             float softmax_scale, const float* out) {
  if (!kv || num_seqs < 0 || max_blocks <= 0 || q_per_seq <= 0) return MSA_ERR_INVALID_ARG;
  if (kv->head_dim != MSA_HEAD_DIM || kv->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (kv->num_heads < 1 || kv->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (num_q_heads != MSA_HEADS_PER_KV * kv->num_heads) return MSA_ERR_UNSUPPORTED;
  if (q_per_seq > MSA_MAX_Q_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (kv->num_pages <= 0 || kv->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (int64_t(max_blocks) * MSA_BLOCK_TOKENS > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return MSA_ERR_INVALID_ARG;
  if (num_seqs == 0) return MSA_OK;
  if (int64_t(num_seqs) * q_per_seq > 65535) return MSA_ERR_UNSUPPORTED;
  if (!k_codes || !k_scales || !v_codes || !v_scales || !q_fp8 || !block_table || !seq_lens || !out)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(k_codes, 15) || misaligned(k_scales, 15) || misaligned(v_codes, 15) ||
      misaligned(v_scales, 15) || misaligned(q_fp8, 15) || misaligned(block_table, 3) ||
      misaligned(seq_lens, 3) || misaligned(out, 15))
    return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// Plan, workspace carving and launches (attention, then the split merge).
template <bool SELECT>
static msa_status run_attn(AttnArgs a, const msa_pool_desc* kv, int32_t num_seqs,
                           int32_t q_per_seq, int32_t num_q_heads, void* workspace,
                           size_t workspace_bytes, hipStream_t s) {
  const int64_t tq = int64_t(num_seqs) * q_per_seq;
  const AttnPlan plan = attn_plan(tq * kv->num_heads, a.num_sel);
  a.slots_per_wg = plan.slots_per_wg;
  a.num_splits = plan.splits;
  if (a.num_splits > 1) {
    const size_t need = msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads, a.num_sel);
    if (!workspace || workspace_bytes < need || misaligned(workspace, 255)) return MSA_ERR_WORKSPACE;
    const size_t rows = size_t(tq) * num_q_heads;
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + align256(rows * a.num_splits * MSA_HEAD_DIM * 4));
  } else {
    a.part_o = nullptr;
    a.part_ml = nullptr;
  }
  const dim3 grid(a.num_splits, kv->num_heads, unsigned(tq));
  if (plan.tok == kBlockTokens)
    hipLaunchKernelGGL((sparse_attn_kernel<kBlockTokens, SELECT>), grid, dim3(64 * kAttnWaves),
                       attn_lds_bytes<kBlockTokens>(), s, a);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<kBlockTokens / kAttnWaves, SELECT>), grid,
                       dim3(64 * kAttnWaves), attn_lds_bytes<kBlockTokens / kAttnWaves>(), s, a);
  if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  if (a.num_splits > 1) {
    hipLaunchKernelGGL(merge_kernel, dim3(unsigned(tq * kv->num_heads)), dim3(256), 0, s,
                       a.part_o, a.part_ml, a.num_splits, a.out);
    if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  }
  return MSA_OK;
}

static AttnArgs base_args(const msa_pool_desc* kv, const uint8_t* k_codes, const uint8_t* k_scales,
                          const uint8_t* v_codes, const uint8_t* v_scales, const uint8_t* q_fp8,
                          int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, int32_t q_per_seq, float softmax_scale,
                          float* out) {
  AttnArgs a{};
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.num_pages = kv->num_pages;
  a.num_kv_heads = kv->num_heads;
  a.q = q_fp8;
  a.num_q_heads = num_q_heads;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.q_per_seq = q_per_seq;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.out = out;
  return a;
}

}  // namespace msa

extern "C" msa_status msa_sparse_attn_decode(const msa_pool_desc* kv, const uint8_t* k_codes,
                                             const uint8_t* k_scales, const uint8_t* v_codes,
                                             const uint8_t* v_scales, const uint8_t* q_fp8,
                                             int32_t num_q_heads, const int32_t* block_table,
                                             int32_t max_blocks, const int32_t* seq_lens,
                                             int32_t num_seqs, int32_t q_per_seq,
                                             const int32_t* sel_ids, int32_t num_sel,
                                             float softmax_scale, float* out, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  using namespace msa;
  msa_status st = check_attn(kv, k_codes, k_scales, v_codes, v_scales, q_fp8, num_q_heads,
                             block_table, max_blocks, seq_lens, num_seqs, q_per_seq, softmax_scale,
                             out);
  if (st != MSA_OK) return st;
  if (num_sel < 1 || num_sel > 64) return MSA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return MSA_OK;
  if (!sel_ids || misaligned(sel_ids, 3)) return MSA_ERR_INVALID_ARG;
  AttnArgs a = base_args(kv, k_codes, k_scales, v_codes, v_scales, q_fp8, num_q_heads, block_table,
                         max_blocks, seq_lens, q_per_seq, softmax_scale, out);
  a.sel_ids = sel_ids;
  a.num_sel = num_sel;
  return run_attn<false>(a, kv, num_seqs, q_per_seq, num_q_heads, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

extern "C" msa_status msa_sparse_attn_select_decode(
    const msa_pool_desc* kv, const uint8_t* k_codes, const uint8_t* k_scales,
    const uint8_t* v_codes, const uint8_t* v_scales, const uint8_t* q_fp8, int32_t num_q_heads,
    const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
    int32_t q_per_seq, const float* block_scores, int32_t topk, int32_t* out_ids,
    float softmax_scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace msa;
  msa_status st = check_attn(kv, k_codes, k_scales, v_codes, v_scales, q_fp8, num_q_heads,
                             block_table, max_blocks, seq_lens, num_seqs, q_per_seq, softmax_scale,
                             out);
  if (st != MSA_OK) return st;
  if (topk != MSA_TOPK) return MSA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return MSA_OK;
  if (!block_scores || misaligned(block_scores, 3) || misaligned(out_ids, 3))
    return MSA_ERR_INVALID_ARG;
  AttnArgs a = base_args(kv, k_codes, k_scales, v_codes, v_scales, q_fp8, num_q_heads, block_table,
                         max_blocks, seq_lens, q_per_seq, softmax_scale, out);
  a.bscore = block_scores;
  a.out_ids = out_ids;
  a.num_sel = MSA_TOPK + 1;
  return run_attn<true>(a, kv, num_seqs, q_per_seq, num_q_heads, workspace, workspace_bytes,
                        static_cast<hipStream_t>(stream));
}
