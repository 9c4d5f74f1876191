// indexer.hip -- msa_indexer_decode: scan the NVFP4 index-key cache, score
// 128-token blocks, and select the top-16 blocks plus the most recent one.
//
// The pages: the indexer still scans the whole history, only with smaller
// reads than K/V (MiniMax-M3.1-Flash serving summary, section "Sparse
// attention still scans an index"); the index cache is NVFP4 and the FP8
// queries force a conversion to FP8 before the QK product (MiniMax-M3.1-Flash
// lands in vLLM on day one, third paragraph); several heads and speculative
// query tokens are batched to fill the matrix units (serving summary,
// section "Parallelize index work across context").
//
// Two kernels. The scan kernel has grid (block chunks, sequences) and one
// wavefront per index-key head; workgroup x of a sequence takes blocks x,
// x + G, x + 2G, ... (G = grid width); with shared prefixes its leading
// rows hold the shared-prefix workgroups (shared_workgroup below), which
// score each shared block once for all the sequences of its group. Per
// 128-token block a wave streams its
// head's 8 KiB of codes and 1 KiB of scales in coalesced 16-byte
// non-temporal loads (lane l: token row 16j + l%16, 32-channel slice l/16),
// turns them into FP8 MFMA operands through the LDS lookup table, and
// multiplies them with the FP8 index queries held in registers:
// A = queries (16 rows = 8 heads x up to 2 query tokens), B = 16 tokens x 128
// channels. The epilogue applies ReLU and the head weights and leaves
// per-token partial scores in LDS; the waves' partials are summed over heads
// and maximised over the block's visible tokens, giving one fp32 block score
// per (query token, block). The selection kernel then picks, per query
// token, the top-16 blocks plus the most recent one.
#include <algorithm>
#include <atomic>
#include <unordered_map>
#include <vector>

#include "msa_nvfp4.h"
#include "nvfp4_tile.h"
#include "topk_select.h"
#include "scan_body.h"

namespace msa {

static_assert(kTopK == MSA_TOPK, "selection size");

__constant__ Fp8Lut kIdxLut = make_fp8_lut();

// One shared-prefix workgroup: block j of group g, one wavefront per index
// head. The block (the group lead's page) is read once and dequantised once
// into registers, then scored against the query tokens of every sequence of
// the group whose block j maps to the same page, two tokens at a time (16
// MFMA rows: token R/8, head R%8 of the wave's 8). The arithmetic per token
// is the regular scan's, in the same order (the same MFMA operands, the
// ReLU-weighted sum of a lane's 4 heads, the head-pair exchange, the sum over
// index heads in head order, the maximum over the visible tokens), so the
// block scores are the values the regular scan would write. LDS from the
// caller: part = [2][H][2][128] floats, lut = 128 table rows.
__device__ __forceinline__ void shared_workgroup(const IndexerArgs& a, int j, int g, float* part,
                                                 uint2* lut) {
  __shared__ int memb[65];  // member sequences of the current chunk of 64, then their count
  const int H = a.num_heads;
  const int Q = a.q_per_seq;
  const int Hq = a.num_q_heads;
  const int tid = int(__builtin_amdgcn_workitem_id_x());
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slice = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // uniform over the workgroup: nothing to do past the group's shared blocks
  if (g >= a.num_groups || j >= min(a.group_blocks[g], a.max_blocks)) return;
  const int lead = a.group_lead[g];
  if (lead < 0 || lead >= a.num_seqs) return;

  for (int i = tid; i < 128; i += 64 * H) lut[i] = make_uint2(kIdxLut.lo[i], kIdxLut.hi[i]);
  const int p = a.block_table[int64_t(lead) * a.max_blocks + j];
  const bool page_ok = p >= 0 && p < a.num_pages;
  TileLoads t;
  issue_loads(t, a.codes + int64_t(wave_u) * kCodePage, a.scales + int64_t(wave_u) * kScalePage,
              p, page_ok, int64_t(H) * kCodePage, int64_t(H) * kScalePage,
              (lane & 15) * kCodeRow + slice * 16, scale_word_offset(slice, lane & 15));
  __syncthreads();  // the lookup table
  v8i kop[8];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const uint32_t sj = tile_scales(t.s, jj);
    kop[jj] = dequant32(t.c[jj], lut[sj & 0x7F], lut[(sj >> 8) & 0x7F]);
  }
  const int part_lane = (lane >> 5) * kBlockTokens + (lane & 31);
  const int part_stride = H * 2 * kBlockTokens;
  int u_all = 0;  // token pairs processed so far (partial buffer parity)
  for (int c0 = 0; c0 < a.num_seqs; c0 += 64) {
    if (c0 > 0) __syncthreads();  // the previous chunk's last reduction has read memb
    // this chunk's members: the sequences of group g whose block j is the
    // lead's page and whose length is valid; each lane of wave 0 tests one
    if (wave_u == 0) {
      const int bb = c0 + lane;
      bool m = false;
      if (bb < a.num_seqs && a.seq_group[bb] == g) {
        const int L = a.seq_lens[bb];
        m = L >= Q && L <= a.max_blocks * kBlockTokens &&
            a.block_table[int64_t(bb) * a.max_blocks + j] == p;
      }
      const uint64_t mask = __ballot(m);
      if (m) memb[__popcll(mask & ((uint64_t(1) << lane) - 1))] = bb;
      if (lane == 0) memb[64] = __popcll(mask);
    }
    __syncthreads();  // memb
    const int T = __builtin_amdgcn_readfirstlane(memb[64]) * Q;  // member query tokens
    for (int u = 0; 2 * u < T; ++u, ++u_all) {
      const int buf = u_all & 1;
      // operands of tokens 2u, 2u + 1: row R of a 16-row group is token
      // 2u + R/8, head R%8 of this wave's index head
      v8i qop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      float wv[4];
      {
        const int R = lane & 15;
        const int tk = 2 * u + (R >> 3);
        if (tk < T) {
          const int bb = memb[tk / Q];
          const int row = bb * Q + tk % Q;
          const uint4* qp = reinterpret_cast<const uint4*>(
              a.q + (int64_t(row) * Hq + wave * kHeadsPerKv + (R & 7)) * kHeadDim + slice * 32);
          qop = q_operand(qp[0], qp[1]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int R2 = 4 * slice + v;
          const int tk2 = 2 * u + (R2 >> 3);
          wv[v] = 0.0f;
          if (tk2 < T) {
            const int bb = memb[tk2 / Q];
            wv[v] = a.w[(int64_t(bb) * Q + tk2 % Q) * Hq + wave * kHeadsPerKv + (R2 & 7)];
          }
        }
      }
      // ReLU-weighted head sums per token, head pairs combined, to LDS
      float* pw = part + buf * part_stride + wave * 2 * kBlockTokens + part_lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float s2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const v4f acc = mfma_fp8_16x16x128(qop, kop[2 * i + e], v4f{0.0f, 0.0f, 0.0f, 0.0f});
          float sc = wv[0] * fmaxf(acc[0], 0.0f);
          sc += wv[1] * fmaxf(acc[1], 0.0f);
          sc += wv[2] * fmaxf(acc[2], 0.0f);
          sc += wv[3] * fmaxf(acc[3], 0.0f);
          s2[e] = sc;
        }
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(s2[0]),
                                                         __float_as_uint(s2[1]), false, false);
        pw[32 * i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      __syncthreads();
      // sum over index heads and maximum over the visible tokens of the
      // pair, by one wavefront
      if (wave_u == u_all % H) {
        const int tk = 2 * u + (lane >> 5);
        int lim = -1;
        int row = 0;
        if (tk < T) {
          const int bb = memb[tk / Q];
          const int L = a.seq_lens[bb];
          row = bb * Q + tk % Q;
          lim = L - Q + tk % Q - j * kBlockTokens;
        }
        const float2 mx = row_pair_max(part + buf * part_stride, 2 * kBlockTokens, H, 0, lim, lane);
        const int rl = __shfl(row, lane * 32, 64);   // lane 0: row of token 2u, lane 1: 2u + 1
        const int ll = __shfl(lim, lane * 32, 64);
        if (lane < 2 && 2 * u + lane < T && ll >= 0)
          a.bscore[int64_t(rl) * a.max_blocks + j] = page_ok ? (lane ? mx.y : mx.x) : 0.0f;
      }
    }
  }
}

// QG: 16-row MFMA groups per index head = ceil(8 * q_per_seq / 16).
// Grid (G, shared_rows + num_seqs + tail_rows): the first shared_rows rows
// are the shared-prefix workgroups (row-major over (group, block)),
// dispatched first so that they run beside the regular scan; row
// shared_rows + b holds the G scan workgroups of sequence b (blocks
// x + G k below tail_first); the last tail_rows rows hold one workgroup per
// remaining block (sequence-major). Workgroups are dispatched in grid order,
// so the short one-block workgroups run last and the chip drains in about
// one block's time instead of one regular workgroup's.
// One block in flight per wave: the next block's loads are issued as soon as
// the current block's codes are consumed, and more resident waves hide the
// latency better than a second register buffer would (measured with 1 and 8
// query tokens).
// SHARED: the launch holds shared-prefix workgroups (msa_indexer_scan_shared);
// their role is compiled only into this form, whose register allocation it
// raises (112 VGPRs against 84 for the plain scan with one query token).
// With one query token the plain form asks for at least five wavefronts per
// SIMD (at most 96 VGPRs); it compiles to 78, six wavefronts. With four row
// groups (5..8 query tokens) it asks for four (at most 128 VGPRs): the four
// accumulators of a tile's products then fit at 126 VGPRs, where the
// unconstrained allocation takes 138 and three wavefronts.
template <int QG, bool SHARED>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(
    QG == 1 && !SHARED ? 5 : (QG == 4 ? 4 : 1))))
void indexer_kernel(const IndexerArgs a) {
  extern __shared__ float part[];  // [2][H][2*QG][128] partial token scores per index head
  __shared__ uint2 lut[128];
  __shared__ ScanList list;
  int y = blockIdx.y;
  if constexpr (SHARED) {
    if (y < a.shared_rows) {
      const int u = y * int(gridDim.x) + int(blockIdx.x);
      shared_workgroup(a, u % a.max_group_blocks, u / a.max_group_blocks, part, lut);
      return;
    }
    y -= a.shared_rows;
  }
  if (y >= a.num_seqs) {
    // the trailing one-block workgroups (uniform over the workgroup)
    const int per_seq = a.max_blocks - a.tail_first;
    const int u = (y - a.num_seqs) * int(gridDim.x) + int(blockIdx.x);
    const int b = u / per_seq;
    if (b >= a.num_seqs) return;
    scan_workgroup<QG, false>(a, a.tail_first + (u - b * per_seq), 1, 1, b, kIdxLut, part, lut,
                              list);
    return;
  }
  scan_workgroup<QG, false>(a, blockIdx.x, gridDim.x, a.blocks_per_wg, y, kIdxLut, part, lut,
                            list);
}

// Selection kernel: one wavefront per query token (topk_select.h).
__global__ __launch_bounds__(64) void select_kernel(const float* __restrict__ bscore,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int max_blocks, int q_per_seq,
                                                    int32_t* __restrict__ out_ids,
                                                    float* __restrict__ out_scores) {
  __shared__ SelectScratch scratch;
  // ids through the builtins: this file is built without IEEE NaN handling,
  // so the device library's id functions are not inlined here, and a called
  // one returns its value in a register the compiler cannot treat as uniform
  // (each buffer load then needed a loop over the descriptor's values)
  const int row = int(__builtin_amdgcn_workgroup_id_x());
  const int lane = int(__builtin_amdgcn_workitem_id_x());
  const float* src = bscore + int64_t(row) * max_blocks;
  float x0[kSelPerLane];
  load_score_chunk(src, max_blocks, 0, lane, x0);  // in flight while the length is read
  const int Q = q_per_seq;
  const int b = row / Q, qi = row - b * Q;
  const int L = seq_lens[b];
  int32_t* ids = out_ids + int64_t(row) * (kTopK + 1);
  float* sc = out_scores ? out_scores + int64_t(row) * (kTopK + 1) : nullptr;
  if (L < Q || L > max_blocks * kBlockTokens) {
    if (lane <= kTopK) {
      ids[lane] = -1;
      if (sc) sc[lane] = 0.0f;
    }
    return;
  }
  const int nb = (L - Q + qi) / kBlockTokens + 1;
  float score;
  const int id = select_blocks(src, max_blocks, nb, x0, scratch, lane, &score);
  if (lane <= kTopK) {
    ids[lane] = id;
    if (sc) sc[lane] = score;
  }
}

}  // namespace msa

namespace msa {

// Host-side checks shared by the indexer entry points.
static msa_status check_indexer_shape(int32_t num_seqs, int32_t q_per_seq, int32_t max_blocks) {
  if (num_seqs < 0 || max_blocks <= 0 || q_per_seq <= 0) return MSA_ERR_INVALID_ARG;
  if (q_per_seq > MSA_MAX_Q_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (int64_t(max_blocks) * MSA_BLOCK_TOKENS > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  if (num_seqs > 65535) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

static bool misaligned(const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) != 0; }

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Shared-prefix groups of a scan (device arrays), or none.
struct SharedGroups {
  const int32_t* seq_group = nullptr;
  const int32_t* group_lead = nullptr;
  const int32_t* group_blocks = nullptr;
  int num_groups = 0;
  int max_group_blocks = 0;
};

// Workgroups of a scan kernel the chip holds at once (occupancy per CU x
// CUs), looked up once per device and kernel form; 0 if unknown.
template <int QG, bool SHARED>
static int64_t resident_of(int threads, size_t lds) {
  int dev = -1, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, indexer_kernel<QG, SHARED>, threads,
                                                   lds) != hipSuccess)
    return 0;
  return int64_t(per_cu) * cus;
}
static int64_t scan_resident_wgs(int qg_pow2, bool shared, int threads, size_t lds) {
  constexpr int kDevs = 64;
  static std::atomic<int64_t> cache[kDevs][3][2][MSA_MAX_HEADS + 1];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  const int qi = qg_pow2 == 1 ? 0 : (qg_pow2 == 2 ? 1 : 2);
  const int h = threads / 64;
  if (h < 1 || h > MSA_MAX_HEADS) return 0;
  std::atomic<int64_t>& slot = cache[dev][qi][shared ? 1 : 0][h];
  int64_t r = slot.load(std::memory_order_relaxed);
  if (r > 0) return r;
  if (qi == 0)
    r = shared ? resident_of<1, true>(threads, lds) : resident_of<1, false>(threads, lds);
  else if (qi == 1)
    r = shared ? resident_of<2, true>(threads, lds) : resident_of<2, false>(threads, lds);
  else
    r = shared ? resident_of<4, true>(threads, lds) : resident_of<4, false>(threads, lds);
  if (r > 0) slot.store(r, std::memory_order_relaxed);
  return r;
}

static msa_status launch_scan(const msa_pool_desc* idx, const uint8_t* idx_codes,
                              const uint8_t* idx_scales, const uint8_t* q_fp8, const float* head_w,
                              int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                              float* block_scores, hipStream_t s,
                              const SharedGroups& sg = SharedGroups()) {
  IndexerArgs a;
  a.codes = idx_codes;
  a.scales = idx_scales;
  a.num_pages = idx->num_pages;
  a.num_heads = idx->num_heads;
  a.q = q_fp8;
  a.w = head_w;
  a.num_q_heads = num_q_heads;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.seq_lens = seq_lens;
  a.q_per_seq = q_per_seq;
  a.bscore = block_scores;
  a.num_seqs = num_seqs;
  const bool shared = sg.num_groups > 0;
  a.seq_group = shared ? sg.seq_group : nullptr;
  a.group_lead = sg.group_lead;
  a.group_blocks = sg.group_blocks;
  a.num_groups = shared ? sg.num_groups : 0;
  a.max_group_blocks = shared ? sg.max_group_blocks : 1;
  const int qg = (MSA_HEADS_PER_KV * q_per_seq + 15) / 16;
  const int qg_pow2 = qg == 1 ? 1 : (qg == 2 ? 2 : 4);
  const size_t lds = size_t(2) * idx->num_heads * (2 * qg_pow2) * MSA_BLOCK_TOKENS * sizeof(float);
  const dim3 block(64 * idx->num_heads);
  const int bpw = scan_blocks_per_wg(num_seqs, max_blocks, qg);
  a.blocks_per_wg = bpw;
  // one-block workgroups for the last blocks of every sequence, about one
  // chip's worth of resident workgroups in all, when the regular grid takes
  // more than one round of the chip (32 x 32K, 1.8 rounds: 54.9 -> 54.1 us)
  int gx = (max_blocks + bpw - 1) / bpw;
  a.tail_first = max_blocks;
  a.tail_rows = 0;
  const int64_t resident = scan_resident_wgs(qg_pow2, shared, int(block.x), lds);
  if (bpw > 1 && resident > 0 && int64_t(num_seqs) * gx > resident) {
    const int64_t tail = std::min<int64_t>((resident + num_seqs - 1) / num_seqs, max_blocks / 2);
    const int g1 = int((max_blocks - tail + bpw - 1) / bpw);
    if (int64_t(g1) * bpw < max_blocks) {
      gx = g1;
      a.tail_first = g1 * bpw;
      a.tail_rows = int((int64_t(num_seqs) * (max_blocks - a.tail_first) + gx - 1) / gx);
    }
  }
  // the shared-prefix workgroups fill whole leading rows of the grid
  const int64_t shared_wgs = int64_t(a.num_groups) * a.max_group_blocks;
  a.shared_rows = int((shared_wgs + gx - 1) / gx);
  if (int64_t(num_seqs) + a.shared_rows + a.tail_rows > 65535) return MSA_ERR_UNSUPPORTED;
  const dim3 grid(gx, num_seqs + a.shared_rows + a.tail_rows);
  if (shared) {
    if (qg_pow2 == 1)
      hipLaunchKernelGGL((indexer_kernel<1, true>), grid, block, lds, s, a);
    else if (qg_pow2 == 2)
      hipLaunchKernelGGL((indexer_kernel<2, true>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((indexer_kernel<4, true>), grid, block, lds, s, a);
  } else {
    if (qg_pow2 == 1)
      hipLaunchKernelGGL((indexer_kernel<1, false>), grid, block, lds, s, a);
    else if (qg_pow2 == 2)
      hipLaunchKernelGGL((indexer_kernel<2, false>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((indexer_kernel<4, false>), grid, block, lds, s, a);
  }
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

static msa_status launch_select(const float* block_scores, const int32_t* seq_lens,
                                int32_t max_blocks, int32_t num_seqs, int32_t q_per_seq,
                                int32_t* out_ids, float* out_scores, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(unsigned(int64_t(num_seqs) * q_per_seq)), dim3(64), 0, s,
                     block_scores, seq_lens, max_blocks, q_per_seq, out_ids, out_scores);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

}  // namespace msa

extern "C" msa_status msa_indexer_scan(const msa_pool_desc* idx, const uint8_t* idx_codes,
                                       const uint8_t* idx_scales, const uint8_t* q_fp8,
                                       const float* head_w, int32_t num_q_heads,
                                       const int32_t* block_table, int32_t max_blocks,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t q_per_seq, float* block_scores, void* stream) {
  using namespace msa;
  if (!idx) return MSA_ERR_INVALID_ARG;
  msa_status st = check_indexer_shape(num_seqs, q_per_seq, max_blocks);
  if (st != MSA_OK) return st;
  if (idx->head_dim != MSA_HEAD_DIM || idx->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (idx->num_heads < 1 || idx->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (num_q_heads != MSA_HEADS_PER_KV * idx->num_heads) return MSA_ERR_UNSUPPORTED;
  if (idx->num_pages <= 0 || idx->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (num_seqs == 0) return MSA_OK;
  if (!idx_codes || !idx_scales || !q_fp8 || !head_w || !block_table || !seq_lens || !block_scores)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(idx_codes, 15) || misaligned(idx_scales, 15) || misaligned(q_fp8, 15) ||
      misaligned(head_w, 3) || misaligned(block_table, 3) || misaligned(seq_lens, 3) ||
      misaligned(block_scores, 3))
    return MSA_ERR_INVALID_ARG;
  return launch_scan(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads, block_table,
                     max_blocks, seq_lens, num_seqs, q_per_seq, block_scores,
                     static_cast<hipStream_t>(stream));
}

extern "C" msa_status msa_indexer_scan_shared(
    const msa_pool_desc* idx, const uint8_t* idx_codes, const uint8_t* idx_scales,
    const uint8_t* q_fp8, const float* head_w, int32_t num_q_heads, const int32_t* block_table,
    int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
    int32_t num_groups, const int32_t* group_lead, const int32_t* group_blocks,
    int32_t max_group_blocks, const int32_t* seq_group, float* block_scores, void* stream) {
  using namespace msa;
  if (!idx) return MSA_ERR_INVALID_ARG;
  msa_status st = check_indexer_shape(num_seqs, q_per_seq, max_blocks);
  if (st != MSA_OK) return st;
  if (idx->head_dim != MSA_HEAD_DIM || idx->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (idx->num_heads < 1 || idx->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (num_q_heads != MSA_HEADS_PER_KV * idx->num_heads) return MSA_ERR_UNSUPPORTED;
  if (idx->num_pages <= 0 || idx->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (num_groups < 0 || num_groups > 65535) return MSA_ERR_INVALID_ARG;
  if (num_groups > 0 && (max_group_blocks < 1 || max_group_blocks > max_blocks))
    return MSA_ERR_INVALID_ARG;
  if (num_seqs == 0) return MSA_OK;
  if (!idx_codes || !idx_scales || !q_fp8 || !head_w || !block_table || !seq_lens || !block_scores)
    return MSA_ERR_INVALID_ARG;
  if (num_groups > 0 && (!group_lead || !group_blocks || !seq_group)) return MSA_ERR_INVALID_ARG;
  if (misaligned(idx_codes, 15) || misaligned(idx_scales, 15) || misaligned(q_fp8, 15) ||
      misaligned(head_w, 3) || misaligned(block_table, 3) || misaligned(seq_lens, 3) ||
      misaligned(block_scores, 3) || misaligned(group_lead, 3) || misaligned(group_blocks, 3) ||
      misaligned(seq_group, 3))
    return MSA_ERR_INVALID_ARG;
  SharedGroups sg;
  sg.seq_group = seq_group;
  sg.group_lead = group_lead;
  sg.group_blocks = group_blocks;
  sg.num_groups = num_groups;
  sg.max_group_blocks = max_group_blocks;
  return launch_scan(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads, block_table, max_blocks,
                     seq_lens, num_seqs, q_per_seq, block_scores,
                     static_cast<hipStream_t>(stream), sg);
}

extern "C" msa_status msa_shared_prefix_groups(const int32_t* block_table, int32_t max_blocks,
                                               const int32_t* seq_lens, int32_t num_seqs,
                                               int32_t q_per_seq, int32_t* group_lead,
                                               int32_t* group_blocks, int32_t* seq_group,
                                               int32_t* num_groups, int32_t* max_group_blocks) {
  if (num_seqs < 0 || max_blocks <= 0 || q_per_seq <= 0) return MSA_ERR_INVALID_ARG;
  if (!num_groups || !max_group_blocks) return MSA_ERR_INVALID_ARG;
  *num_groups = 0;
  *max_group_blocks = 0;
  if (num_seqs == 0) return MSA_OK;
  if (!block_table || !seq_lens || !group_lead || !group_blocks || !seq_group)
    return MSA_ERR_INVALID_ARG;
  // candidate groups: sequences with a valid length keyed by their first
  // page (pages < 0 map nothing), in the order of their first member
  std::unordered_map<int32_t, int32_t> by_first;
  std::vector<std::vector<int32_t>> members;
  for (int32_t b = 0; b < num_seqs; ++b) {
    seq_group[b] = -1;
    const int32_t L = seq_lens[b];
    if (L < q_per_seq || int64_t(L) > int64_t(max_blocks) * MSA_BLOCK_TOKENS) continue;
    const int32_t p0 = block_table[int64_t(b) * max_blocks];
    if (p0 < 0) continue;
    auto it = by_first.find(p0);
    if (it == by_first.end()) {
      by_first.emplace(p0, int32_t(members.size()));
      members.push_back({b});
    } else {
      members[it->second].push_back(b);
    }
  }
  // a group of two or more shares the longest run of leading blocks whose
  // pages are the same (and mapped) in every member, within every member's
  // own blocks; the lead is its first member
  int32_t ng = 0, mgb = 0;
  for (const auto& m : members) {
    if (m.size() < 2) continue;
    const int32_t lead = m[0];
    const int32_t* lt = block_table + int64_t(lead) * max_blocks;
    int32_t n = max_blocks;
    for (int32_t b : m) n = std::min(n, (seq_lens[b] + MSA_BLOCK_TOKENS - 1) / MSA_BLOCK_TOKENS);
    int32_t run = 0;
    while (run < n && lt[run] >= 0) ++run;
    for (size_t i = 1; i < m.size() && run > 0; ++i) {
      const int32_t* bt = block_table + int64_t(m[i]) * max_blocks;
      int32_t k = 0;
      while (k < run && bt[k] == lt[k]) ++k;
      run = k;
    }
    if (run == 0) continue;
    group_lead[ng] = lead;
    group_blocks[ng] = run;
    for (int32_t b : m) seq_group[b] = ng;
    mgb = std::max(mgb, run);
    ++ng;
  }
  *num_groups = ng;
  *max_group_blocks = mgb;
  return MSA_OK;
}

extern "C" msa_status msa_indexer_select(const float* block_scores, const int32_t* seq_lens,
                                         int32_t max_blocks, int32_t num_seqs, int32_t q_per_seq,
                                         int32_t topk, int32_t* out_ids, float* out_scores,
                                         void* stream) {
  using namespace msa;
  msa_status st = check_indexer_shape(num_seqs, q_per_seq, max_blocks);
  if (st != MSA_OK) return st;
  if (topk != MSA_TOPK) return MSA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return MSA_OK;
  if (!block_scores || !seq_lens || !out_ids) return MSA_ERR_INVALID_ARG;
  if (misaligned(block_scores, 3) || misaligned(seq_lens, 3) || misaligned(out_ids, 3) ||
      misaligned(out_scores, 3))
    return MSA_ERR_INVALID_ARG;
  return launch_select(block_scores, seq_lens, max_blocks, num_seqs, q_per_seq, out_ids,
                       out_scores, static_cast<hipStream_t>(stream));
}

extern "C" size_t msa_indexer_workspace_bytes(int32_t num_seqs, int32_t q_per_seq,
                                              int32_t max_blocks) {
  if (num_seqs <= 0 || q_per_seq <= 0 || max_blocks <= 0) return 0;
  return msa::align256(size_t(num_seqs) * q_per_seq * max_blocks * 4);
}

namespace msa {

// Host checks of msa_indexer_decode's arguments other than the workspace.
static msa_status check_decode(const msa_pool_desc* idx, const uint8_t* idx_codes,
                               const uint8_t* idx_scales, const uint8_t* q_fp8,
                               const float* head_w, int32_t num_q_heads,
                               const int32_t* block_table, int32_t max_blocks,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                               int32_t topk, const int32_t* out_ids, const float* out_scores) {
  if (!idx) return MSA_ERR_INVALID_ARG;
  msa_status st = check_indexer_shape(num_seqs, q_per_seq, max_blocks);
  if (st != MSA_OK) return st;
  if (topk != MSA_TOPK) return MSA_ERR_UNSUPPORTED;
  if (idx->head_dim != MSA_HEAD_DIM || idx->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (idx->num_heads < 1 || idx->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (num_q_heads != MSA_HEADS_PER_KV * idx->num_heads) return MSA_ERR_UNSUPPORTED;
  if (idx->num_pages <= 0 || idx->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (num_seqs == 0) return MSA_OK;
  if (!idx_codes || !idx_scales || !q_fp8 || !head_w || !block_table || !seq_lens || !out_ids)
    return MSA_ERR_INVALID_ARG;
  if (misaligned(idx_codes, 15) || misaligned(idx_scales, 15) || misaligned(q_fp8, 15) ||
      misaligned(head_w, 3) || misaligned(block_table, 3) || misaligned(seq_lens, 3) ||
      misaligned(out_ids, 3) || misaligned(out_scores, 3))
    return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// The block scores of msa_indexer_decode_noalloc live in this array instead
// of a caller's workspace: one copy per GPU the library runs on, resident
// until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) float scratch[MSA_NOALLOC_MAX_SCORES];

constexpr int kMaxDevices = 64;
static std::atomic<float*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first
// call for that device; two threads racing here store the same address).
static msa_status scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MSA_ERR_HIP;
    p = static_cast<float*>(q);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MSA_OK;
}

}  // namespace msa

extern "C" msa_status msa_indexer_decode(const msa_pool_desc* idx, const uint8_t* idx_codes,
                                         const uint8_t* idx_scales, const uint8_t* q_fp8,
                                         const float* head_w, int32_t num_q_heads,
                                         const int32_t* block_table, int32_t max_blocks,
                                         const int32_t* seq_lens, int32_t num_seqs,
                                         int32_t q_per_seq, int32_t topk, int32_t* out_ids,
                                         float* out_scores, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  using namespace msa;
  msa_status st = check_decode(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads,
                               block_table, max_blocks, seq_lens, num_seqs, q_per_seq, topk,
                               out_ids, out_scores);
  if (st != MSA_OK || num_seqs == 0) return st;
  const size_t need = msa_indexer_workspace_bytes(num_seqs, q_per_seq, max_blocks);
  if (!workspace || workspace_bytes < need || misaligned(workspace, 255)) return MSA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* scores = static_cast<float*>(workspace);
  st = launch_scan(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads, block_table, max_blocks,
                   seq_lens, num_seqs, q_per_seq, scores, s);
  if (st != MSA_OK) return st;
  return launch_select(scores, seq_lens, max_blocks, num_seqs, q_per_seq, out_ids, out_scores, s);
}

extern "C" msa_status msa_indexer_decode_noalloc(const msa_pool_desc* idx,
                                                 const uint8_t* idx_codes,
                                                 const uint8_t* idx_scales, const uint8_t* q_fp8,
                                                 const float* head_w, int32_t num_q_heads,
                                                 const int32_t* block_table, int32_t max_blocks,
                                                 const int32_t* seq_lens, int32_t num_seqs,
                                                 int32_t q_per_seq, int32_t topk,
                                                 int32_t* out_ids, float* out_scores,
                                                 void* stream) {
  using namespace msa;
  msa_status st = check_decode(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads,
                               block_table, max_blocks, seq_lens, num_seqs, q_per_seq, topk,
                               out_ids, out_scores);
  if (st != MSA_OK || num_seqs == 0) return st;
  if (int64_t(num_seqs) * q_per_seq * max_blocks > int64_t(MSA_NOALLOC_MAX_SCORES))
    return MSA_ERR_WORKSPACE;
  float* scores = nullptr;
  st = scratch_address(&scores);
  if (st != MSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_scan(idx, idx_codes, idx_scales, q_fp8, head_w, num_q_heads, block_table, max_blocks,
                   seq_lens, num_seqs, q_per_seq, scores, s);
  if (st != MSA_OK) return st;
  return launch_select(scores, seq_lens, max_blocks, num_seqs, q_per_seq, out_ids, out_scores, s);
}
