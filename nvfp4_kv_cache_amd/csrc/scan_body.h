// scan_body.h -- one workgroup of the index scan (msa_indexer_scan and the
// one-launch decode step): stream this workgroup's 128-token blocks of the
// NVFP4 index-key cache, convert them to FP8 through the lookup table,
// multiply them with the FP8 index queries on the matrix cores, and write
// one fp32 score per (query token, block): the maximum over the block's
// visible tokens of the ReLU-weighted sum over the query heads
// (MiniMax-M3.1-Flash serving summary, sections "Sparse attention still
// scans an index" and "Parallelize index work across context";
// MiniMax-M3.1-Flash lands in vLLM on day one, third paragraph).
#pragma once

#include "msa_nvfp4.h"
#include "nvfp4_tile.h"

namespace msa {

struct IndexerArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t num_pages;
  int num_heads;  // index-key heads = wavefronts per workgroup
  const uint8_t* q;
  const float* w;
  int num_q_heads;
  const int32_t* block_table;
  int max_blocks;
  const int32_t* seq_lens;
  int q_per_seq;
  int blocks_per_wg;
  float* bscore;       // [num_seqs * q_per_seq][max_blocks]
  int num_seqs;
  // shared prefixes (seq_group null: none). Block j of sequence b belongs to
  // the shared pass, and not to the regular scan, when g = seq_group[b] is a
  // group (0 <= g < num_groups), j < min(group_blocks[g], max_blocks), the
  // lead l = group_lead[g] is a sequence of the batch, and block_table[b][j]
  // equals block_table[l][j]: the same page, read and dequantised once for
  // every sequence of the group
  const int32_t* seq_group;     // [num_seqs] group of each sequence, -1: none
  const int32_t* group_lead;    // [num_groups] sequence whose pages define the group
  const int32_t* group_blocks;  // [num_groups] leading blocks the group shares
  int num_groups;
  int max_group_blocks;         // >= every group_blocks entry, <= max_blocks
  int shared_rows;              // leading grid rows of shared-prefix workgroups
  // trailing rows of one-block workgroups: blocks tail_first .. max_blocks-1
  // of every sequence (tail_rows 0: none; the regular workgroups then cover
  // every block)
  int tail_first;
  int tail_rows;
};

constexpr int kMaxBlocksPerWg = 8;  // blocks per scan workgroup (page list size)

// The blocks a scan workgroup scores: physical page (-1: outside the pool),
// logical block, and how many.
struct ScanList {
  int page[kMaxBlocksPerWg];
  int blk[kMaxBlocksPerWg];
  int count;
};

// The lead sequence of the shared prefix that covers block j of sequence b
// (the shared pass scores that block when b's page equals the lead's), or -1.
__device__ __forceinline__ int shared_lead(const IndexerArgs& a, int b, int j) {
  if (!a.seq_group) return -1;
  const int g = a.seq_group[b];
  if (g < 0 || g >= a.num_groups || j >= min(a.group_blocks[g], a.max_blocks)) return -1;
  const int lead = a.group_lead[g];
  return (lead >= 0 && lead < a.num_seqs) ? lead : -1;
}

// One block's worth of this wave's loads: 8 tiles x 16 code bytes and the
// 16-byte scale word (2 scale bytes per tile) per lane.
struct TileLoads {
  uint4 c[8];
  uint4 s;
};

// This wave's loads of one block. `live` (uniform) false stands for an
// absent block (past the workgroup's count, or an unmapped page): the
// descriptors then hold no records, every lane receives zeros and nothing is
// read. There is no branch, so the wait the compiler places before a block's
// first use covers that block's loads only, not the next block's issued
// after them.
// The descriptors over one block's code and scale rows of this wave's head.
struct BlockRsrc {
  __amdgpu_buffer_rsrc_t codes, scales;
};
__device__ __forceinline__ BlockRsrc block_rsrc(const uint8_t* codes_w, const uint8_t* scales_w,
                                                int page, bool live, int64_t page_codes,
                                                int64_t page_scales) {
  const int64_t p = live ? page : 0;
  return BlockRsrc{tile_rsrc(codes_w + p * page_codes, live ? kCodePage : 0),
                   tile_rsrc(scales_w + p * page_scales, live ? kScalePage : 0)};
}
__device__ __forceinline__ void issue_loads(TileLoads& t, const uint8_t* codes_w,
                                            const uint8_t* scales_w, int page, bool live,
                                            int64_t page_codes, int64_t page_scales,
                                            uint32_t code_lane, uint32_t scale_lane) {
  const BlockRsrc r = block_rsrc(codes_w, scales_w, page, live, page_codes, page_scales);
#pragma unroll
  for (int j = 0; j < 8; ++j) t.c[j] = load_tile16(r.codes, code_lane, j * 16 * kCodeRow);
  t.s = load_tile16(r.scales, scale_lane, 0);
}

// Block maxima of two query rows r0, r0 + 1 of a partial-score buffer
// part[h][row][t] (rows of 128 floats, head stride hs floats): per token the
// sum over heads 0 .. H-1 in head order, then the maximum, starting from 0,
// over the tokens t <= lim of each row. Lane (row - r0) * 32 + t / 4 sums
// tokens t .. t + 3 with 16-byte LDS reads; lim is the lane's row's last
// visible token in the block (< 0: none). Returns both maxima (uniform).
__device__ __forceinline__ float2 row_pair_max(const float* part, int hs, int H, int r0, int lim,
                                               int lane) {
  const int t0 = 4 * (lane & 31);
  float m = 0.0f;
  if (t0 <= lim) {
    const float* pt = part + (r0 + (lane >> 5)) * kBlockTokens + t0;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int h = 0; h < H; ++h) {
      const float4 v = *reinterpret_cast<const float4*>(pt + h * hs);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    m = fmaxf(fmaxf(m, s.x), t0 + 1 <= lim ? s.y : 0.0f);
    m = fmaxf(m, fmaxf(t0 + 2 <= lim ? s.z : 0.0f, t0 + 3 <= lim ? s.w : 0.0f));
  }
  // m >= 0: maxima of the bit patterns, per 32-lane half
  const uint32_t v = row16_max_u32(__float_as_uint(m));
  const uint32_t a0 = __builtin_amdgcn_readlane(int(v), 15), a1 = __builtin_amdgcn_readlane(int(v), 31);
  const uint32_t a2 = __builtin_amdgcn_readlane(int(v), 47), a3 = __builtin_amdgcn_readlane(int(v), 63);
  return make_float2(__uint_as_float(max(a0, a1)), __uint_as_float(max(a2, a3)));
}

// QG: 16-row MFMA groups per index head = ceil(8 * q_per_seq / 16).
// One block in flight per wave: the next block's loads are issued as soon as
// the current block's codes are consumed, and more resident waves hide the
// latency better than a second register buffer would (measured with 1 and 8
// query tokens).
// Blocks per scan workgroup for num_seqs sequences of up to max_blocks
// blocks and qg 16-row MFMA groups per index head. Halved while the grid
// would not cover the chip several times over. Measured with one query
// token (cold launches, us, with the trailing one-block workgroups): a few
// long sequences (8 x 256K) 94.1-94.3 at 2, 95.2-96.0 at 3, 97.0 at 4,
// 105.3 at 1; 32 x 32K 54.2-54.8 at 3, 54.0 at 4, 54.8-55.5 at 2; many
// sequences of mixed length (45 requests, 30K..210K), where much of the
// grid bound is empty, 233-235 at 8 and 248-252 at 2. The host knows only
// the grid bound num_seqs x max_blocks and max_blocks. With
// 5..8 query tokens a workgroup's blocks cost four times the arithmetic and
// the chip holds about 1,024 workgroups at once (120 VGPRs, 33 KB of LDS
// each): halving stops at that grid. Measured at 16 x 64K with 8 query
// tokens: 8 blocks per workgroup (1,024 workgroups) 66.6 us, 4 (2,048)
// 70.4 us, 2 79.1 us.
inline int scan_blocks_per_wg(int64_t num_seqs, int64_t max_blocks, int qg) {
  int bpw = (qg == 1 && num_seqs * max_blocks <= 32768) ? (max_blocks >= 1024 ? 2 : 3) : 8;
  const int64_t min_grid = qg >= 4 ? 1024 : 2048;
  while (bpw > 1 && num_seqs * ((max_blocks + bpw - 1) / bpw) < min_grid) bpw >>= 1;
  return bpw;
}

// One scan workgroup of sequence b, one wavefront per index-key head: the
// blocks x, x + G, x + 2G, ... (at most `count`, below the sequence's last
// block). LDS from the caller: part = [2][H][2*QG][128] floats, lut = 128
// table rows, the block list. COHERENT: the block scores are stored at
// device scope (write-through), for a consumer in the same launch.
template <int QG, bool COHERENT>
__device__ __forceinline__ void scan_workgroup(const IndexerArgs& a, int x, int G, int count,
                                               int b, const Fp8Lut& lut_src, float* part,
                                               uint2* lut, ScanList& list) {

  const int H = a.num_heads;
  const int Q = a.q_per_seq;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int slice = lane >> 4;  // 32-channel slice of the reduction dimension
  constexpr int QR = 2 * QG;    // query-token rows of the partial buffer

  for (int i = threadIdx.x; i < 128; i += blockDim.x) lut[i] = make_uint2(lut_src.lo[i], lut_src.hi[i]);

  const int L = a.seq_lens[b];
  const bool seq_ok = L >= Q && L <= a.max_blocks * kBlockTokens;
  const int nb_last = seq_ok ? (L - 1) / kBlockTokens + 1 : 0;
  // neighbouring workgroups take neighbouring blocks (x, x + 1, ...), so
  // the workgroups running at any moment read neighbouring pages; a block
  // of a shared prefix whose page is the group lead's is left to the shared
  // pass. Wave 0 builds the list (at most 8 blocks, one lane each).
  const int total = nb_last > x ? min(count, (nb_last - x + G - 1) / G) : 0;
  const int64_t qrow0 = int64_t(b) * Q;
  const int Hq = a.num_q_heads;
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const int j = x + t * G;
    bool keep = t < total;
    int p = -1;
    if (keep) {
      p = a.block_table[int64_t(b) * a.max_blocks + j];
      const int lead = shared_lead(a, b, j);
      if (lead >= 0 && a.block_table[int64_t(lead) * a.max_blocks + j] == p) keep = false;
    }
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int pos = __popcll(m & ((uint64_t(1) << t) - 1));
      list.page[pos] = (p >= 0 && p < a.num_pages) ? p : -1;
      list.blk[pos] = j;
    }
    if (t == 0) list.count = __popcll(m);
  }

  // Query operands (rows: query token R/8, head wave*8 + R%8) and weights.
  v8i qop[QG];
  float wv[QG][4];
#pragma unroll
  for (int rg = 0; rg < QG; ++rg) {
    const int R = 16 * rg + (lane & 15);
    const int qi = R >> 3;
    if (qi < Q) {
      const uint4* qp = reinterpret_cast<const uint4*>(
          a.q + ((qrow0 + qi) * Hq + wave * kHeadsPerKv + (R & 7)) * kHeadDim + slice * 32);
      qop[rg] = q_operand(qp[0], qp[1]);
    } else {
      qop[rg] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int R2 = 16 * rg + 4 * slice + v;
      const int qi2 = R2 >> 3;
      wv[rg][v] = qi2 < Q ? a.w[(qrow0 + qi2) * Hq + wave * kHeadsPerKv + (R2 & 7)] : 0.0f;
    }
  }
  __syncthreads();

  const int64_t page_codes = int64_t(H) * kCodePage;
  const int64_t page_scales = int64_t(H) * kScalePage;
  // this wave's head within a page (uniform), and the lane's offsets in a tile
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint8_t* codes_w = a.codes + int64_t(wave_u) * kCodePage;
  const uint8_t* scales_w = a.scales + int64_t(wave_u) * kScalePage;
  const uint32_t code_lane = (lane & 15) * kCodeRow + slice * 16;
  const uint32_t scale_lane = scale_word_offset(slice, lane & 15);
  const int count_u = __builtin_amdgcn_readfirstlane(list.count);
  // descriptors of the k-th block of the list (none past its end)
  auto rsrc_of = [&](int k) {
    const int page = __builtin_amdgcn_readfirstlane(list.page[min(k, kMaxBlocksPerWg - 1)]);
    return block_rsrc(codes_w, scales_w, page, k < count_u && page >= 0, page_codes, page_scales);
  };
  const int part_stride = H * QR * kBlockTokens;
  // an MFMA result lane l holds query token 2rg + l/32, heads
  // 4*((l/16)&1) .. +3 of the index head's 8, token 16j + l%16; lanes l and
  // l^16 swap halves so that each writes the 8-head sum of one token,
  // 32i + l%32, for the pair j = 2i, 2i+1
  const int part_lane = (lane >> 5) * kBlockTokens + (lane & 31);

  // ROLL (two or more MFMA row groups, a long computation per tile): as soon
  // as tile j is converted, its registers take the next block's tile j, so
  // the next block's loads go out one by one while this block is computed.
  // With one row group the next block's loads go out after the block: that
  // form compiles to 78 VGPRs (six wavefronts per SIMD), and the rolling
  // one, at 82 (five), measured 1.6 us slower at 8 x 256K (forced to six
  // wavefronts it spilled and took 9 us more). With 8 query tokens the
  // rolling form measured 1.3-5 us faster at 16 x 64K.
  constexpr bool ROLL = QG > 1;
  // dequantise, multiply, apply ReLU and weights; per-head partials to LDS.
  // sw: this block's scale word; nx: the next block's descriptors (ROLL).
  auto compute = [&](TileLoads& t, const uint4& sw, const BlockRsrc& nx, int buf) {
    float* pw = part + buf * part_stride + wave * QR * kBlockTokens + part_lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s2[2][QG];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = 2 * i + e;
        const uint32_t sj = tile_scales(sw, j);
        const v8i kop = dequant32(t.c[j], lut[sj & 0x7F], lut[(sj >> 8) & 0x7F]);
        if constexpr (ROLL) t.c[j] = load_tile16(nx.codes, code_lane, j * 16 * kCodeRow);
        // the tile's QG products go out back to back, each into its own
        // accumulator, before their epilogues (with the epilogue after each
        // product, the compiler gave all of them one accumulator and the
        // products waited for each other's epilogues: measured 2% slower
        // with 8 query tokens)
        v4f acc[QG];
#pragma unroll
        for (int rg = 0; rg < QG; ++rg)
          acc[rg] = mfma_fp8_16x16x128(qop[rg], kop, v4f{0.0f, 0.0f, 0.0f, 0.0f});
        if constexpr (QG > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rg = 0; rg < QG; ++rg) {
          float s = wv[rg][0] * fmaxf(acc[rg][0], 0.0f);
          s += wv[rg][1] * fmaxf(acc[rg][1], 0.0f);
          s += wv[rg][2] * fmaxf(acc[rg][2], 0.0f);
          s += wv[rg][3] * fmaxf(acc[rg][3], 0.0f);
          s2[e][rg] = s;
        }
      }
#pragma unroll
      for (int rg = 0; rg < QG; ++rg) {
        // v_permlane16_swap: the odd rows of the first operand trade places
        // with the even rows of the second, so an even-row lane ends with
        // its own j = 2i partial and its partner's, an odd-row lane with
        // both j = 2i+1 partials (heads 0-3 first, as in the unpaired sum)
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2[0][rg]),
                                                         __float_as_uint(s2[1][rg]), false, false);
        pw[2 * rg * kBlockTokens + 32 * i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Sum the heads, maximise over the block's visible tokens and store the
  // block score, one query-token pair per wavefront (waves take pairs w,
  // w + H, ...).
  const int pairs = (Q + 1) >> 1;
  auto reduce_part = [&](int k, int buf) {
    const int blk = list.blk[k];
    const bool page_ok = list.page[k] >= 0;
    for (int u = wave_u; u < pairs; u += H) {
      const int qi = 2 * u + (lane >> 5);
      const int lim = qi < Q ? L - Q + qi - blk * kBlockTokens : -1;
      const float2 mx = row_pair_max(part + buf * part_stride, QR * kBlockTokens, H, 2 * u, lim, lane);
      const int q = 2 * u + lane;
      if (lane < 2 && q < Q && blk * kBlockTokens <= L - Q + q)
      {
        if constexpr (COHERENT)
          __hip_atomic_store(&a.bscore[(qrow0 + q) * a.max_blocks + blk],
                             page_ok ? (lane ? mx.y : mx.x) : 0.0f, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          a.bscore[(qrow0 + q) * a.max_blocks + blk] = page_ok ? (lane ? mx.y : mx.x) : 0.0f;
      }
    }
  };
  // One register buffer, the scale word loaded before the tiles (the
  // scheduling barriers keep that order and keep the compiler from hoisting
  // loads into a second buffer), so each wait counts only the loads issued
  // after the one it waits for. The next block's loads overlap the rest of
  // the block (ROLL), the barrier and the reduction.
  TileLoads t;
  auto load_block = [&](const BlockRsrc& r) {
    t.s = load_tile16(r.scales, scale_lane, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      t.c[j] = load_tile16(r.codes, code_lane, j * 16 * kCodeRow);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  load_block(rsrc_of(0));
  for (int k = 0; k < count_u; ++k) {
    const BlockRsrc nx = rsrc_of(k + 1);
    if constexpr (ROLL) {
      const uint4 sw = t.s;
      t.s = load_tile16(nx.scales, scale_lane, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(t, sw, nx, k & 1);
    } else {
      compute(t, t.s, nx, k & 1);
      __builtin_amdgcn_sched_barrier(0);
      load_block(nx);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    reduce_part(k, k & 1);
  }
}

}  // namespace msa
