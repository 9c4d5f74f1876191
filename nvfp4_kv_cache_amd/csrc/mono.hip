// mono.hip -- msa_decode_mono: the whole decode step (index scan, block
// selection, sparse attention) in one kernel launch, for low concurrency.
//
// The pages: at low concurrency a separate mono-kernel strategy reduces
// launches, and one kernel arrangement need not suit every regime
// (MiniMax-M3.1-Flash serving summary, sections "AMD uses different
// conversion and communication mechanisms" and "Keep capacity, layer, and
// system results separate").
//
// A small step is latency-bound: every stage is a chain of dependent memory
// round trips, and the two-launch path (scan, then selection + attention
// with the split merge) runs them back to back. Here the attention does not
// wait for the selection. One 1-D grid holds three kinds of workgroup, in this order:
//   1. scan workgroups (scan_body.h), scan_per_seq per sequence, which store
//      their block scores at device scope and count themselves in the
//      sequence's arrival counter;
//   2. block workgroups (attn_workgroup.inc, kAttnEvery), one per (block j, KV head,
//      query token) for every block j < max_blocks, which compute block j's
//      attention partial (m, l, o) for the 8 query heads of the KV head
//      whether or not the selection will take it, store it at device scope
//      and count themselves in the pair's arrival counter;
//   3. merge workgroups, one per (query token, KV head), which wait for the
//      sequence's scan, select the 16 + 1 blocks from the scores
//      (topk_select.h) while the partials are still being computed, wait for
//      the pair's partials and merge only the selected blocks' partials by
//      log-sum-exp, in ascending block order.
// So the scan and the attention run side by side, and the selection and the
// merge are the only steps after the scan. The price is attention over every
// block instead of 17 (max_blocks x 73,728 bytes of K/V per sequence), which
// is why the entry point bounds the grid (low concurrency, short contexts:
// query tokens x 4 KV heads x max_blocks <= 1,024).
//
// The values are those of the two-launch path: the scan and the block
// partials are the same code, the selection sees the same scores, and the
// merge combines the same partials in the same order, so the ids and the
// output match msa_indexer_scan + msa_sparse_attn_select_decode bit for bit
// when the latter runs one workgroup per selected block (at most 384
// (query token, KV head, slot) units).
//
// Ordering across workgroups of one launch: a producer's data stores are
// device-scope (write-through, coherent across the XCDs' L2 caches); each
// wave waits for its stores to complete before the workgroup's arrival is
// counted with a device-scope atomic; a consumer polls the counters with
// device-scope loads and reads the data with device-scope loads. Atomics on
// one address are serialised at the memory side, so each arrival count is
// spread over kSubCounters counters on separate 64-byte lines (producer i
// adds to counter i % kSubCounters) and the consumer waits for their sum.
// Workgroups are dispatched in grid order and only merge workgroups (last in
// the grid) wait, for workgroups dispatched before them, so the waits end;
// each wait is still bounded (kMonoWaitTicks), and a wait that times out
// leaves zero output, ids -1 and a nonzero error word instead of hanging.
// Every counter is reset by its last consumer (a pair's counters by its
// merge workgroup, a sequence's scan counters by the last of its merge
// workgroups to pass its wait), so every call leaves them zero.
#include "msa_nvfp4.h"
#include "nvfp4_tile.h"
#include "topk_select.h"
#include "scan_body.h"
#include "attn_body.h"

namespace msa {

__constant__ Fp8Lut kMonoLut = make_fp8_lut();

// Bound on a merge workgroup's wait: 20 ms of the 100 MHz real-time clock.
constexpr uint64_t kMonoWaitTicks = 2000000;
// Bound on block workgroups per launch: T_q x KV heads x max_blocks. Past
// it, attending every block costs more than the launches it saves: measured
// against the multi-launch step (one query token): 512 workgroups (1 x 16K)
// 14.1 vs 16.1 us, 1,024 (1 x 32K, 2 x 16K) 16.2 vs 16.6 and 16.5 vs 16.9 us,
// 1,536 (1 x 48K) 21.4 vs 17.6 us, 2,048 (1 x 64K) 25.3 vs 17.9 us.
constexpr int64_t kMonoMaxBlockWgs = 1024;
// Counters per arrival count, and the word stride between them (64 bytes).
constexpr int kSubCounters = 8;
constexpr int kCounterStride = 16;
constexpr int kCountWords = kSubCounters * kCounterStride;  // one arrival count

struct MonoArgs {
  IndexerArgs s;     // scan (s.bscore: the block scores)
  AttnArgs t;        // block partials (t.num_splits = max_blocks)
  int scan_per_seq;  // scan workgroups per sequence
  int n_scan;        // scan workgroups
  int n_block;       // block workgroups
  int num_seqs;
  int pairs;         // T_q x KV heads
  uint32_t* scan_cnt;   // [num_seqs][kCountWords] scan arrivals
  uint32_t* pair_cnt;   // [pairs][kCountWords] block-partial arrivals
  uint32_t* readers;    // [num_seqs][kCounterStride] merge workgroups past their wait
  uint32_t* err;        // error word: the workspace's last 32-bit word
  int32_t* out_ids;  // [T_q][17] or null
};

// One wavefront: wait until the kSubCounters counters of an arrival count
// sum to target (lane i < kSubCounters reads counter i); bounded, false on
// timeout.
__device__ __forceinline__ bool wait_count(const uint32_t* cnt, uint32_t target, int lane) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t v = lane < kSubCounters
                           ? __hip_atomic_load(cnt + lane * kCounterStride, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)
                           : 0u;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kSubCounters; ++i) sum += __builtin_amdgcn_readlane(v, i);
    if (sum >= target) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kMonoWaitTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Zero the kSubCounters counters of an arrival count (lanes < kSubCounters).
__device__ __forceinline__ void clear_count(uint32_t* cnt, int lane) {
  if (lane < kSubCounters)
    __hip_atomic_store(cnt + lane * kCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count producer i of an arrival count once every wave's stores have completed.
__device__ __forceinline__ void arrive(uint32_t* cnt, int i) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's device-scope stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(cnt + (i % kSubCounters) * kCounterStride, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Merge workgroup of (query token qt, KV head kh).
__device__ __forceinline__ void merge_pair(const MonoArgs& m, int qt, int kh, uint8_t* smem) {
  __shared__ int slot[kTopK + 1];
  const AttnArgs& t = m.t;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int Q = t.q_per_seq;
  const int b = qt / Q, qi = qt - b * Q;
  const int pair = qt * t.num_kv_heads + kh;
  // wave 0: wait for the sequence's scan, select (the pair's block
  // partials are still being computed meanwhile), then wait for the partials
  if (wave == 0) {
    uint32_t* scnt = m.scan_cnt + int64_t(b) * kCountWords;
    uint32_t* pcnt = m.pair_cnt + int64_t(pair) * kCountWords;
    bool ok = wait_count(scnt, uint32_t(m.scan_per_seq), lane);
    int sel = -1;
    if (ok) {
      const int L = t.seq_lens[b];
      if (L >= Q && L <= t.max_blocks * kBlockTokens) {
        const float* row = m.s.bscore + int64_t(qt) * t.max_blocks;
        float x0[kSelPerLane];
        load_score_chunk<true>(row, t.max_blocks, 0, lane, x0);
        float score;
        sel = select_blocks<true>(row, t.max_blocks, (L - Q + qi) / kBlockTokens + 1, x0,
                                  *reinterpret_cast<SelectScratch*>(smem), lane, &score);
      }
      // the sequence's scan counters go to the last of its merge workgroups
      // past this point
      uint32_t prev = 0;
      if (lane == 0)
        prev = __hip_atomic_fetch_add(m.readers + int64_t(b) * kCounterStride, 1u,
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == uint32_t(Q * t.num_kv_heads - 1)) {
        clear_count(scnt, lane);
        if (lane == 0)
          __hip_atomic_store(m.readers + int64_t(b) * kCounterStride, 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
      ok = wait_count(pcnt, uint32_t(t.max_blocks), lane);
      // every partial of the pair has arrived: its counters are this
      // workgroup's alone to reset
      if (ok) clear_count(pcnt, lane);
    }
    if (!ok) {
      sel = -1;
      if (lane == 0) __hip_atomic_store(m.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane <= kTopK) {
      slot[lane] = sel;
      if (m.out_ids && kh == 0) m.out_ids[int64_t(qt) * (kTopK + 1) + lane] = sel;
    }
  }
  __syncthreads();
  // thread: head tid / 32 of this KV head, channels 4 (tid % 32) .. + 3
  const int64_t row = int64_t(qt) * t.num_q_heads + kh * kHeadsPerKv + (tid >> 5);
  const int pd = (tid & 31) * 4;
  const int64_t nsp = t.num_splits;
  const auto ro = partial_rsrc(t.part_o), rm = partial_rsrc(t.part_ml);
  *reinterpret_cast<float4*>(t.out + row * kHeadDim + pd) =
      merge_row(kTopK + 1, [&](int k, float4& v, float2& ml) {
        const int s = slot[k];  // selected block (-1: none)
        if (s < 0) return false;
        v = load_device_scope4(ro, uint32_t(((row * nsp + s) * kHeadDim + pd) * 4));
        ml = load_device_scope2(rm, uint32_t((row * nsp + s) * 8));
        return true;
      });
}

template <int QG>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mono_kernel(
    const MonoArgs m) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int id = blockIdx.x;
  if (id < m.n_scan) {
    __shared__ uint2 lut[128];
    __shared__ ScanList list;
    const int b = id / m.scan_per_seq;
    const int x = id - b * m.scan_per_seq;
    scan_workgroup<QG, true>(m.s, x, m.scan_per_seq, m.s.blocks_per_wg, b, kMonoLut,
                             reinterpret_cast<float*>(smem), lut, list);
    arrive(m.scan_cnt + int64_t(b) * kCountWords, x);
  } else if (id < m.n_scan + m.n_block) {
    const int u = id - m.n_scan;
    const int j = u % m.t.max_blocks;
    const int p = u / m.t.max_blocks;  // qt * KV heads + kh
    {
      constexpr int TOK = kBlockTokens / kAttnWaves;
      constexpr int MODE = kAttnEvery;
      const int sp = j, kh = p % m.t.num_kv_heads, qt = p / m.t.num_kv_heads;
      const AttnArgs& a = m.t;
      const Fp8Lut& lut_src = kMonoLut;
#include "attn_workgroup.inc"
    }
    arrive(m.pair_cnt + int64_t(p) * kCountWords, j);
  } else {
    const int p = id - m.n_scan - m.n_block;
    merge_pair(m, p / m.t.num_kv_heads, p % m.t.num_kv_heads, smem);
  }
}

inline size_t mono_align256(size_t x) { return (x + 255) & ~size_t(255); }
inline bool mono_misaligned(const void* p, uintptr_t m) {
  return (reinterpret_cast<uintptr_t>(p) & m) != 0;
}

// Workspace layout: block scores, partial o, partial (m, l), counters.
struct MonoLayout {
  size_t scores, part_o, part_ml, sync, total;
};
inline MonoLayout mono_layout(int64_t tq, int64_t num_q_heads, int64_t max_blocks, int64_t num_seqs) {
  MonoLayout l;
  const int64_t rows = tq * num_q_heads;
  const int64_t pairs = tq * (num_q_heads / kHeadsPerKv);
  l.scores = 0;
  l.part_o = mono_align256(size_t(tq * max_blocks) * 4);
  l.part_ml = l.part_o + mono_align256(size_t(rows * max_blocks * kHeadDim) * 4);
  l.sync = l.part_ml + mono_align256(size_t(rows * max_blocks * 2) * 4);
  l.total = l.sync + mono_align256(size_t((num_seqs + pairs) * kCountWords +
                                          num_seqs * kCounterStride + 1) * 4);
  return l;
}

}  // namespace msa

extern "C" size_t msa_decode_mono_workspace_bytes(int32_t num_seqs, int32_t q_per_seq,
                                                  int32_t num_q_heads, int32_t max_blocks) {
  if (num_seqs <= 0 || q_per_seq <= 0 || num_q_heads <= 0 || max_blocks <= 0) return 0;
  return msa::mono_layout(int64_t(num_seqs) * q_per_seq, num_q_heads, max_blocks, num_seqs).total;
}

extern "C" msa_status msa_decode_mono(
    const msa_pool_desc* idx, const uint8_t* idx_codes, const uint8_t* idx_scales,
    const uint8_t* q_idx_fp8, const float* head_w, const msa_pool_desc* kv,
    const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v_codes,
    const uint8_t* v_scales, const uint8_t* q_fp8, int32_t num_q_heads,
    const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
    int32_t q_per_seq, int32_t topk, int32_t* out_ids, float softmax_scale, float* out,
    void* workspace, size_t workspace_bytes, void* stream) {
  using namespace msa;
  if (!idx || !kv || num_seqs < 0 || max_blocks <= 0 || q_per_seq <= 0) return MSA_ERR_INVALID_ARG;
  if (idx->head_dim != MSA_HEAD_DIM || idx->block_tokens != MSA_BLOCK_TOKENS ||
      kv->head_dim != MSA_HEAD_DIM || kv->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (topk != MSA_TOPK) return MSA_ERR_UNSUPPORTED;
  // one 256-thread workgroup shape for all three roles: 4 index-key heads
  // (one wavefront each in the scan), 4 KV heads, 32 query heads
  if (idx->num_heads != 4 || kv->num_heads != 4 || num_q_heads != MSA_HEADS_PER_KV * 4)
    return MSA_ERR_UNSUPPORTED;
  if (q_per_seq > MSA_MAX_Q_PER_SEQ) return MSA_ERR_UNSUPPORTED;
  if (idx->num_pages <= 0 || idx->num_pages > 0x7FFFFFFF || kv->num_pages <= 0 ||
      kv->num_pages > 0x7FFFFFFF)
    return MSA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f) || softmax_scale > 1e30f) return MSA_ERR_INVALID_ARG;
  const int64_t tq = int64_t(num_seqs) * q_per_seq;
  if (tq * kv->num_heads * max_blocks > kMonoMaxBlockWgs) return MSA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return MSA_OK;
  if (!idx_codes || !idx_scales || !q_idx_fp8 || !head_w || !k_codes || !k_scales || !v_codes ||
      !v_scales || !q_fp8 || !block_table || !seq_lens || !out)
    return MSA_ERR_INVALID_ARG;
  if (mono_misaligned(idx_codes, 15) || mono_misaligned(idx_scales, 15) ||
      mono_misaligned(q_idx_fp8, 15) || mono_misaligned(head_w, 3) ||
      mono_misaligned(k_codes, 15) || mono_misaligned(k_scales, 15) ||
      mono_misaligned(v_codes, 15) || mono_misaligned(v_scales, 15) ||
      mono_misaligned(q_fp8, 15) || mono_misaligned(block_table, 3) ||
      mono_misaligned(seq_lens, 3) || mono_misaligned(out_ids, 3) || mono_misaligned(out, 15))
    return MSA_ERR_INVALID_ARG;
  const MonoLayout lay = mono_layout(tq, num_q_heads, max_blocks, num_seqs);
  if (!workspace || workspace_bytes < lay.total || mono_misaligned(workspace, 255))
    return MSA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);

  MonoArgs m{};
  IndexerArgs& s = m.s;
  s.codes = idx_codes;
  s.scales = idx_scales;
  s.num_pages = idx->num_pages;
  s.num_heads = idx->num_heads;
  s.q = q_idx_fp8;
  s.w = head_w;
  s.num_q_heads = num_q_heads;
  s.block_table = block_table;
  s.max_blocks = max_blocks;
  s.seq_lens = seq_lens;
  s.q_per_seq = q_per_seq;
  s.bscore = reinterpret_cast<float*>(ws + lay.scores);
  s.num_seqs = num_seqs;
  s.seq_group = nullptr;
  s.num_groups = 0;
  s.max_group_blocks = 1;
  s.shared_rows = 0;
  // blocks per scan workgroup: the standalone scan's rule
  const int qg = (MSA_HEADS_PER_KV * q_per_seq + 15) / 16;
  const int bpw = scan_blocks_per_wg(num_seqs, max_blocks, qg);
  s.blocks_per_wg = bpw;

  AttnArgs& t = m.t;
  t.k_codes = k_codes;
  t.k_scales = k_scales;
  t.v_codes = v_codes;
  t.v_scales = v_scales;
  t.num_pages = kv->num_pages;
  t.num_kv_heads = kv->num_heads;
  t.q = q_fp8;
  t.num_q_heads = num_q_heads;
  t.block_table = block_table;
  t.max_blocks = max_blocks;
  t.seq_lens = seq_lens;
  t.q_per_seq = q_per_seq;
  t.num_sel = max_blocks;
  t.slots_per_wg = 1;
  t.num_splits = max_blocks;
  t.scale_log2 = softmax_scale * 1.4426950408889634f;
  t.part_o = reinterpret_cast<float*>(ws + lay.part_o);
  t.part_ml = reinterpret_cast<float*>(ws + lay.part_ml);
  t.out = out;

  m.scan_per_seq = (max_blocks + bpw - 1) / bpw;
  m.n_scan = int(int64_t(num_seqs) * m.scan_per_seq);
  m.n_block = int(tq * kv->num_heads * max_blocks);
  m.num_seqs = num_seqs;
  m.pairs = int(tq * kv->num_heads);
  m.scan_cnt = reinterpret_cast<uint32_t*>(ws + lay.sync);
  m.pair_cnt = m.scan_cnt + int64_t(num_seqs) * kCountWords;
  m.readers = m.pair_cnt + int64_t(m.pairs) * kCountWords;
  m.err = reinterpret_cast<uint32_t*>(ws + lay.total - 4);
  m.out_ids = out_ids;

  const int qg_pow2 = qg == 1 ? 1 : (qg == 2 ? 2 : 4);
  const size_t scan_lds = size_t(2) * idx->num_heads * (2 * qg_pow2) * MSA_BLOCK_TOKENS * 4;
  size_t lds = scan_lds;
  lds = lds > attn_lds_bytes<kBlockTokens / kAttnWaves>() ? lds : attn_lds_bytes<kBlockTokens / kAttnWaves>();
  lds = lds > sizeof(SelectScratch) ? lds : sizeof(SelectScratch);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(unsigned(m.n_scan + m.n_block + m.pairs)), block(256);
  if (qg_pow2 == 1)
    hipLaunchKernelGGL((mono_kernel<1>), grid, block, lds, st, m);
  else if (qg_pow2 == 2)
    hipLaunchKernelGGL((mono_kernel<2>), grid, block, lds, st, m);
  else
    hipLaunchKernelGGL((mono_kernel<4>), grid, block, lds, st, m);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
