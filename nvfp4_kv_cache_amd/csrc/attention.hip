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
// waves merge through LDS, and with several splits the last split of each
// (query token, KV head) pair to finish merges the splits' (m, l, o) by
// log-sum-exp, counted in the workspace. Per block a wave:
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
#include "attn_body.h"

namespace msa {

__constant__ Fp8Lut kAttnLut = make_fp8_lut();

// One workgroup (attn_workgroup.inc) per (split, KV head, query token).
// kSelects: the workgroup selects the blocks itself from the indexer's block
// scores; otherwise the caller's ids are used.
// Two wavefronts per SIMD (two workgroups per CU), held by the attribute:
// with one allowed, the compiler moved registers to AGPRs (212 + 36) and
// workgroups no longer ran two to a CU (measured with per-workgroup time
// stamps), and the quarter-block form spilled at three.
template <int TOK, bool kSelects>
__global__ __launch_bounds__(64 * kAttnWaves)
__attribute__((amdgpu_waves_per_eu(2))) void sparse_attn_kernel(const AttnArgs a) {
  constexpr int MODE = kSelects ? kAttnSelect : kAttnIds;
  const int sp = blockIdx.x, kh = blockIdx.y, qt = blockIdx.z;
  const Fp8Lut& lut_src = kAttnLut;
#include "attn_workgroup.inc"
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool misaligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) != 0; }

// Launch plan for `pairs` (query token, KV head) pairs and num_sel slots.
// Few pairs (pairs * num_sel <= kSharedMaxWgs): one workgroup per selected
// block, its four wavefronts sharing the block (32 tokens each), so the
// serial work per wavefront is a quarter block. Measured against whole
// blocks per wavefront at 17 slots: 2.3 us faster per step at 4 pairs, 1.5 us
// at 16, 0.4 us slower at 32 (more workgroups than the chip runs evenly).
// Otherwise whole blocks per wavefront: R slots per wavefront and
// ceil(num_sel / 4R) splits per pair. The chip holds kResidentWgs of these
// workgroups at once (two per CU at the kernel's ~210 VGPRs). Among the R
// whose grid fits in one round, the one with the shortest chain wins: R
// blocks per wavefront at ~3 time units each with one workgroup per CU
// (a wavefront alone on its SIMD; phase stamps: ~3.2 us per block) or ~5
// with two (two wavefronts share a SIMD: ~5.5 us), plus ~1.5 for the split
// merge; ties go to fewer splits. When none fits, one split per pair (R =
// ceil(num_sel / 4)). Measured at 17 slots, us per launch (R = 1 / 2 / 3 /
// 5): 32 pairs 15.3 / 17.9 / - / -; 128 pairs 27.9 / 23.4 / 22.0 / 23.9;
// 180 pairs - / 29.5 / 27.6 / 24.4; 512 pairs - / - / 51.7 / 38.9; and
// with an earlier build 96 pairs 19.9 / 24.3 / 23.7 / 27.6, 160 pairs
// 30.4 / 25.2 / 29.8 / 27.8, 192 pairs 31.8 / 31.3 / 30.1 / 28.1: the rule
// picks the fastest in each.
constexpr int64_t kSharedMaxWgs = 384;
constexpr int64_t kResidentWgs = 512;
constexpr int64_t kCUs = kResidentWgs / 2;
struct AttnPlan {
  int tok;           // tokens of a block per wavefront: 32 or 128
  int slots_per_wg;  // selected slots per workgroup
  int splits;        // workgroups per pair
};
inline AttnPlan attn_plan(int64_t pairs, int num_sel) {
  if (pairs * num_sel <= kSharedMaxWgs) return AttnPlan{kBlockTokens / kAttnWaves, 1, num_sel};
  auto splits = [&](int r) { return (num_sel + kAttnWaves * r - 1) / (kAttnWaves * r); };
  const int r_max = (num_sel + kAttnWaves - 1) / kAttnWaves;  // one split
  int R = r_max;
  int64_t best = -1;
  for (int r = 1; r <= r_max; ++r) {
    const int64_t wgs = pairs * splits(r);
    if (wgs > kResidentWgs) continue;
    const int64_t cost = int64_t(r) * (wgs <= kCUs ? 30 : 50) + (splits(r) > 1 ? 15 : 0);
    if (best < 0 || cost < best || (cost == best && splits(r) < splits(R))) {
      best = cost;
      R = r;
    }
  }
  return AttnPlan{kBlockTokens, kAttnWaves * R, splits(R)};
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
  const size_t pairs = size_t(num_seqs) * q_per_seq * kv_heads;
  return msa::align256(rows * splits * MSA_HEAD_DIM * 4) + msa::align256(rows * splits * 2 * 4) +
         msa::align256(pairs * 4);
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

// Plan, workspace carving and the launch (the last split of each pair merges).
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
    const size_t o_bytes = align256(rows * a.num_splits * MSA_HEAD_DIM * 4);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(ws + o_bytes);
    a.split_cnt = reinterpret_cast<uint32_t*>(ws + o_bytes + align256(rows * a.num_splits * 2 * 4));
  } else {
    a.part_o = nullptr;
    a.part_ml = nullptr;
    a.split_cnt = nullptr;
  }
  const dim3 grid(a.num_splits, kv->num_heads, unsigned(tq));
  if (plan.tok == kBlockTokens)
    hipLaunchKernelGGL((sparse_attn_kernel<kBlockTokens, SELECT>), grid, dim3(64 * kAttnWaves),
                       attn_lds_bytes<kBlockTokens>(), s, a);
  else
    hipLaunchKernelGGL((sparse_attn_kernel<kBlockTokens / kAttnWaves, SELECT>), grid,
                       dim3(64 * kAttnWaves), attn_lds_bytes<kBlockTokens / kAttnWaves>(), s, a);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
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
