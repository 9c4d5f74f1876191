// attention.hip -- msa_sparse_attn_decode: exact GQA attention of each query
// token over the visible tokens of its selected blocks, with the NVFP4 K and
// V pages converted to FP8 through the lookup table before the products.
//
// The pages: main attention runs over the roughly 2,048 keys of the selected
// blocks, exactly (MiniMax-M3.1-Flash serving summary, section "Sparse
// attention still scans an index"); the NVFP4 cache is converted to FP8
// because the query stays FP8 (MiniMax-M3.1-Flash lands in vLLM on day one,
// third paragraph).
//
// Grid (splits, KV heads, query tokens). A workgroup (4 wavefronts) takes a
// run of selected blocks of one query token and one KV head (its 8 query
// heads). Per block: every wave dequantises 2 of the 8 16-token K tiles
// straight into FP8 MFMA operands and multiplies them with the query
// (A = 8 heads, B = 16 tokens); it dequantises the same tokens' V rows into
// LDS as fp32. The softmax runs online in base 2 with fp32 state, and P x V
// is accumulated in fp32 on the vector ALUs. Each split writes (m, l, o);
// the last split of a (query token, KV head) to finish merges them.
#include "msa_nvfp4.h"
#include "nvfp4_tile.h"

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
  const int32_t* sel_ids;
  int num_sel;
  int blocks_per_split;
  int num_splits;
  float scale_log2;  // softmax_scale * log2(e)
  float* part_o;     // [T_q * Hq][num_splits][128]
  float* part_ml;    // [T_q * Hq][num_splits][2]
  float* out;
};

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kAttnThreads = 256;

__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(const AttnArgs a) {
  __shared__ uint2 lut[128];
  __shared__ float vs[kBlockTokens][kHeadDim];   // dequantised V of one block
  __shared__ float zs[kHeadsPerKv][kBlockTokens];  // logits, then probabilities
  __shared__ float alpha_s[kHeadsPerKv];
  __shared__ float s_m[kHeadsPerKv][64], s_l[kHeadsPerKv][64];

  const int qt = blockIdx.z, kh = blockIdx.y, sp = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, slice = lane >> 4;
  const int Q = a.q_per_seq;
  const int b = qt / Q, qi = qt % Q;
  const int Hq = a.num_q_heads;

  for (int i = tid; i < 128; i += kAttnThreads) lut[i] = make_uint2(kAttnLut.lo[i], kAttnLut.hi[i]);

  const int L = a.seq_lens[b];
  const bool seq_ok = L >= Q && L <= a.max_blocks * kBlockTokens;
  const int pos = L - Q + qi;

  // query operand: rows 0..7 = the 8 query heads of this KV head
  v8i qop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  if ((lane & 15) < kHeadsPerKv) {
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + (int64_t(qt) * Hq + kh * kHeadsPerKv + (lane & 15)) * kHeadDim + slice * 32);
    qop = q_operand(qp[0], qp[1]);
  }
  // softmax state of heads 2*wave, 2*wave+1 (wave-uniform)
  float m_run[2] = {-__builtin_huge_valf(), -__builtin_huge_valf()};
  float l_run[2] = {0.0f, 0.0f};
  // P x V accumulator: head tid/32, channels 4*(tid%32) .. +3
  const int ph = tid >> 5, pd = (tid & 31) * 4;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  __syncthreads();

  const int64_t page_codes = int64_t(a.num_kv_heads) * kCodePage;
  const int64_t page_scales = int64_t(a.num_kv_heads) * kScalePage;
  const int lane_code = (lane & 15) * kCodeRow + slice * 16;
  const int lane_scale = (lane & 15) * kScaleRow + slice * 2;

  const int s0 = sp * a.blocks_per_split;
  const int s1 = min(a.num_sel, s0 + a.blocks_per_split);
  for (int si = s0; si < s1; ++si) {
    const int blk = a.sel_ids[int64_t(qt) * a.num_sel + si];
    bool ok = seq_ok && blk >= 0 && blk < a.max_blocks && blk * kBlockTokens <= pos;
    int page = -1;
    if (ok) {
      page = a.block_table[int64_t(b) * a.max_blocks + blk];
      ok = page >= 0 && page < a.num_pages;
    }
    if (!ok) continue;  // uniform over the workgroup
    const int ntok = min(kBlockTokens, pos + 1 - blk * kBlockTokens);
    const int64_t head_code = int64_t(page) * page_codes + int64_t(kh) * kCodePage + lane_code;
    const int64_t head_scale = int64_t(page) * page_scales + int64_t(kh) * kScalePage + lane_scale;

#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * wave + jj;
      const int t = 16 * j + (lane & 15);
      const uint4 kc = *reinterpret_cast<const uint4*>(a.k_codes + head_code + j * 16 * kCodeRow);
      const uint32_t ks = *reinterpret_cast<const uint16_t*>(a.k_scales + head_scale + j * 16 * kScaleRow);
      const uint4 vc = *reinterpret_cast<const uint4*>(a.v_codes + head_code + j * 16 * kCodeRow);
      const uint32_t vsc = *reinterpret_cast<const uint16_t*>(a.v_scales + head_scale + j * 16 * kScaleRow);
      const v8i kop = dequant32(kc, lut[ks & 0x7F], lut[(ks >> 8) & 0x7F]);
      const v4f z = mfma_fp8_16x16x128(qop, kop, v4f{0.0f, 0.0f, 0.0f, 0.0f});
      if (lane < 32) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          zs[4 * slice + v][t] = t < ntok ? z[v] * a.scale_log2 : -__builtin_huge_valf();
      }
      // V: 32 channels of token t, restored to natural channel order
      // (dequant32 yields channels 0,2,4,6 then 1,3,5,7 of each run of 8)
      const v8i vop = dequant32(vc, lut[vsc & 0x7F], lut[(vsc >> 8) & 0x7F]);
      float* dst = &vs[t][slice * 32];
      const bool live = t < ntok;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2f e01 = __builtin_amdgcn_cvt_pk_f32_fp8(vop[2 * u], false);     // ch 0, 2
        const v2f e23 = __builtin_amdgcn_cvt_pk_f32_fp8(vop[2 * u], true);      // ch 4, 6
        const v2f o01 = __builtin_amdgcn_cvt_pk_f32_fp8(vop[2 * u + 1], false); // ch 1, 3
        const v2f o23 = __builtin_amdgcn_cvt_pk_f32_fp8(vop[2 * u + 1], true);  // ch 5, 7
        const float4 lo = live ? make_float4(e01.x, o01.x, e01.y, o01.y) : make_float4(0, 0, 0, 0);
        const float4 hi = live ? make_float4(e23.x, o23.x, e23.y, o23.y) : make_float4(0, 0, 0, 0);
        *reinterpret_cast<float4*>(dst + 8 * u) = lo;
        *reinterpret_cast<float4*>(dst + 8 * u + 4) = hi;
      }
    }
    __syncthreads();
    // online softmax for heads 2*wave, 2*wave+1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int h = 2 * wave + hh;
      const float z0 = zs[h][lane], z1 = zs[h][lane + 64];
      const float m_new = fmaxf(m_run[hh], wave_max(fmaxf(z0, z1)));
      const float p0 = exp2f(z0 - m_new), p1 = exp2f(z1 - m_new);
      zs[h][lane] = p0;
      zs[h][lane + 64] = p1;
      const float alpha = exp2f(m_run[hh] - m_new);
      l_run[hh] = l_run[hh] * alpha + wave_sum(p0 + p1);
      m_run[hh] = m_new;
      if (lane == 0) alpha_s[h] = alpha;
    }
    __syncthreads();
    {
      const float al = alpha_s[ph];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= al;
      for (int t = 0; t < ntok; ++t) {
        const float p = zs[ph][t];
        const float4 v = *reinterpret_cast<const float4*>(&vs[t][pd]);
        acc[0] += p * v.x;
        acc[1] += p * v.y;
        acc[2] += p * v.z;
        acc[3] += p * v.w;
      }
    }
    __syncthreads();
  }

  const int64_t row = int64_t(qt) * Hq + kh * kHeadsPerKv;  // first query head row
  // per-head (m, l) of this wave's two heads go through LDS to the P x V threads
  if (lane == 0) {
    s_m[2 * wave][0] = m_run[0];
    s_m[2 * wave + 1][0] = m_run[1];
    s_l[2 * wave][0] = l_run[0];
    s_l[2 * wave + 1][0] = l_run[1];
  }
  __syncthreads();
  if (a.num_splits == 1) {
    const float l = s_l[ph][0];
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    *reinterpret_cast<float4*>(a.out + (row + ph) * kHeadDim + pd) =
        make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    return;
  }
  float* po = a.part_o + ((row + ph) * a.num_splits + sp) * kHeadDim + pd;
  *reinterpret_cast<float4*>(po) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  if ((tid & 31) == 0) {
    float* pm = a.part_ml + ((row + ph) * a.num_splits + sp) * 2;
    pm[0] = s_m[ph][0];
    pm[1] = s_l[ph][0];
  }
}

// Merge kernel: one workgroup per (query token, KV head); thread (h, 4 ch)
// combines the splits' (m, l, o) by log-sum-exp. Every (m, l) and every
// partial o is fetched with independent loads.
__global__ __launch_bounds__(kAttnThreads) void merge_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_ml,
                                                             int num_splits, float* __restrict__ out) {
  __shared__ float s_m[kHeadsPerKv][64], s_l[kHeadsPerKv][64];
  const int tid = threadIdx.x;
  const int64_t row = int64_t(blockIdx.x) * kHeadsPerKv;  // first query head row
  for (int i = tid; i < kHeadsPerKv * num_splits; i += kAttnThreads) {
    const int h = i / num_splits, sidx = i - h * num_splits;
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((row + h) * num_splits + sidx) * 2);
    s_m[h][sidx] = ml.x;
    s_l[h][sidx] = ml.y;
  }
  __syncthreads();
  const int ph = tid >> 5, pd = (tid & 31) * 4;
  float M = -__builtin_huge_valf();
  for (int sidx = 0; sidx < num_splits; ++sidx) M = fmaxf(M, s_m[ph][sidx]);
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f}, den = 0.0f;
  if (M != -__builtin_huge_valf()) {
    const float* po = part_o + (row + ph) * num_splits * kHeadDim + pd;
    for (int s0 = 0; s0 < num_splits; s0 += 8) {
      float4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        v[k] = s0 + k < num_splits ? *reinterpret_cast<const float4*>(po + (s0 + k) * kHeadDim)
                                   : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (s0 + k >= num_splits) break;
        const float ms = s_m[ph][s0 + k];
        const float f = ms == -__builtin_huge_valf() ? 0.0f : exp2f(ms - M);
        den += f * s_l[ph][s0 + k];
        o[0] += f * v[k].x;
        o[1] += f * v[k].y;
        o[2] += f * v[k].z;
        o[3] += f * v[k].w;
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  *reinterpret_cast<float4*>(out + (row + ph) * kHeadDim + pd) =
      make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Split count: enough workgroups to cover the chip, never more than num_sel.
inline void attn_splits(int64_t tq_kv, int num_sel, int* bps, int* nsplit) {
  int want = int((2048 + tq_kv - 1) / tq_kv);
  want = want < 1 ? 1 : (want > num_sel ? num_sel : want);
  *bps = (num_sel + want - 1) / want;
  *nsplit = (num_sel + *bps - 1) / *bps;
}

}  // namespace msa

extern "C" size_t msa_attn_workspace_bytes(int32_t num_seqs, int32_t q_per_seq,
                                           int32_t num_q_heads, int32_t num_sel) {
  if (num_seqs <= 0 || q_per_seq <= 0 || num_q_heads <= 0 || num_sel <= 0) return 0;
  const size_t rows = size_t(num_seqs) * q_per_seq * num_q_heads;
  // partial o and partial (m, l) for up to num_sel splits
  return msa::align256(rows * num_sel * MSA_HEAD_DIM * 4) + msa::align256(rows * num_sel * 2 * 4);
}

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
  if (!kv || num_seqs < 0 || max_blocks <= 0 || q_per_seq <= 0) return MSA_ERR_INVALID_ARG;
  if (kv->head_dim != MSA_HEAD_DIM || kv->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (kv->num_heads < 1 || kv->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (num_q_heads != MSA_HEADS_PER_KV * kv->num_heads) return MSA_ERR_UNSUPPORTED;
  if (q_per_seq > MSA_MAX_Q_PER_SEQ || num_sel < 1 || num_sel > 64) return MSA_ERR_UNSUPPORTED;
  if (kv->num_pages <= 0 || kv->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (int64_t(max_blocks) * MSA_BLOCK_TOKENS > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return MSA_ERR_INVALID_ARG;
  if (num_seqs == 0) return MSA_OK;
  if (int64_t(num_seqs) * q_per_seq > 65535) return MSA_ERR_UNSUPPORTED;
  if (!k_codes || !k_scales || !v_codes || !v_scales || !q_fp8 || !block_table || !seq_lens ||
      !sel_ids || !out)
    return MSA_ERR_INVALID_ARG;
  auto mis = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) != 0; };
  if (mis(k_codes, 15) || mis(k_scales, 15) || mis(v_codes, 15) || mis(v_scales, 15) ||
      mis(q_fp8, 15) || mis(block_table, 3) || mis(seq_lens, 3) || mis(sel_ids, 3) || mis(out, 15))
    return MSA_ERR_INVALID_ARG;
  const size_t need = msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads, num_sel);
  if (!workspace || workspace_bytes < need || mis(workspace, 255)) return MSA_ERR_WORKSPACE;

  const int64_t tq = int64_t(num_seqs) * q_per_seq;
  const size_t rows = size_t(tq) * num_q_heads;
  AttnArgs a;
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
  a.sel_ids = sel_ids;
  a.num_sel = num_sel;
  attn_splits(tq * kv->num_heads, num_sel, &a.blocks_per_split, &a.num_splits);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  char* ws = static_cast<char*>(workspace);
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + align256(rows * num_sel * MSA_HEAD_DIM * 4));
  a.out = out;
  const dim3 grid(a.num_splits, kv->num_heads, unsigned(tq));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sparse_attn_kernel, grid, dim3(kAttnThreads), 0, s, a);
  if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  if (a.num_splits > 1) {
    hipLaunchKernelGGL(merge_kernel, dim3(unsigned(tq * kv->num_heads)), dim3(kAttnThreads), 0, s,
                       a.part_o, a.part_ml, a.num_splits, out);
    if (hipGetLastError() != hipSuccess) return MSA_ERR_HIP;
  }
  return MSA_OK;
}
