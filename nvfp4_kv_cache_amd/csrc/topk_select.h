// topk_select.h -- block selection of one query token by one wavefront:
// the 16 best blocks among 0..nb-2 by (score descending, block ascending),
// plus the most recent block nb-1, in ascending block order (MiniMax-M3.1-Flash
// serving summary, section "Sparse attention still scans an index": top-16
// blocks plus the recent block, about 2,048 keys).
//
// No sort and no workgroup barrier. A block's key is (score bits << 32 |
// ~block): scores are non-negative, so their fp32 bit patterns order like
// the values, and the low word makes every key distinct and breaks ties
// toward the lower block. Steps:
//   1. lane l holds the scores of blocks l, l+64, ..., l+64*31 of a chunk of
//      2,048 (one chunk in registers; longer contexts loop over chunks) and
//      their maximum;
//   2. theta = the 16th largest of the 64 lane maxima (a radix select with
//      wavefront votes): the 16 lanes holding the largest maxima each own a
//      block scoring >= theta, so at least 16 candidates reach theta and the
//      top-16 are among them;
//   3. the candidates >= theta (typically 16..25) are compacted into LDS at
//      offsets from a DPP prefix sum of per-lane hit counts and ranked exactly
//      by counting against broadcast LDS reads; with more than 64 of them
//      (many equal scores) 16 rounds of wavefront arg-max take over. With at
//      most 64 candidates in all, steps 1-3 reduce to ranking them all
//      directly (measured: 1 x 4K step 16.0 -> 14.5 us);
//   4. each winner finds its place in ascending block order by counting; the
//      recent block goes last.
#pragma once

#include "nvfp4_tile.h"

namespace msa {

constexpr int kTopK = 16;
constexpr int kSelPerLane = 32;               // scores per lane per chunk
constexpr int kSelChunk = 64 * kSelPerLane;   // 2,048 candidates per chunk

struct __align__(16) SelectScratch {
  uint32_t stage[kSelChunk];  // the current chunk's score bits, [k][lane]
  uint64_t cand[64];          // compacted candidates (keys)
  uint64_t win[kTopK];
  int32_t id[kTopK];
  float score[kTopK];
  int32_t page[kTopK];
};

__device__ __forceinline__ uint32_t score_bits(float s) { return __float_as_uint(s > 0.0f ? s : 0.0f); }
__device__ __forceinline__ uint64_t make_key(uint32_t bits, int j) {
  return (uint64_t(bits) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(j));
}
__device__ __forceinline__ int key_block_id(uint64_t k) { return int(0xFFFFFFFFu - uint32_t(k)); }
__device__ __forceinline__ float key_score_value(uint64_t k) { return __uint_as_float(uint32_t(k >> 32)); }

// Buffer-load cache policy for scores written earlier in the same launch:
// device scope (sc1), so the load is coherent across the XCDs' L2 caches.
constexpr int kDeviceScopeLoad = 16;

// One score entry; COHERENT: a device-scope load (see kDeviceScopeLoad).
template <bool COHERENT>
__device__ __forceinline__ float load_score(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// One chunk of a query token's block scores: lane l gets entries
// c0 + l + 64 k. The loads go through a buffer descriptor over the row
// (row_len entries), with one 32-bit lane offset and the stride of k in the
// scalar offset operand: nothing is predicated, so all 32 loads are in flight
// at once, no per-element 64-bit address is formed, and no vector register
// holds a per-k offset. The descriptor's range check covers the lane offset
// plus the scalar offset (an in-bounds probe on gfx950: a load whose scalar
// offset alone passes the record count returns 0), so entries past the row
// read as 0 and touch no memory; they are masked by index later anyway.
// COHERENT: device-scope loads.
template <bool COHERENT = false>
__device__ __forceinline__ void load_score_chunk(const float* row, int row_len, int c0, int lane,
                                                 float (&x)[kSelPerLane]) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(row), 0, row_len * int(sizeof(float)), 0x00020000);
  const uint32_t off = uint32_t(c0 + lane) * uint32_t(sizeof(float));
#pragma unroll
  for (int k = 0; k < kSelPerLane; ++k)
    x[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         r, off, 64 * k * int(sizeof(float)),
                                         COHERENT ? kDeviceScopeLoad : 0));
}

// Inclusive prefix sum over the wavefront: DPP row shifts inside rows of 16
// lanes (out-of-row lanes read 0), then the totals of the preceding rows.
__device__ __forceinline__ int wave_inclusive_sum(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// theta of a selection: the largest x, truncated below bit 11, with at
// least 16 lanes of the wavefront holding m >= x (radix select on the bit
// patterns, two bits at a time from the top with three wavefront votes).
__device__ __forceinline__ uint32_t select_theta(uint32_t m) {
  uint32_t theta = 0;
#pragma unroll
  for (int bit = 29; bit >= 11; bit -= 2) {
    const uint32_t t1 = theta | (1u << bit), t2 = theta | (2u << bit), t3 = theta | (3u << bit);
    const int c1 = __popcll(__ballot(m >= t1));
    const int c2 = __popcll(__ballot(m >= t2));
    const int c3 = __popcll(__ballot(m >= t3));
    theta = c3 >= kTopK ? t3 : (c2 >= kTopK ? t2 : (c1 >= kTopK ? t1 : theta));
  }
  return theta;
}

// Selection for one query token with nb visible blocks whose scores are
// row[0 .. nb-1] (row_len >= nb readable entries); x0 holds chunk 0 as
// load_score_chunk(row, row_len, 0, lane, x0) returns it. Every lane of the
// wavefront must call it. Lane l < 17 receives the l-th selected block
// (ascending; the recent block last when nb > 17) and its score; other lanes,
// and lanes past nb when nb <= 17, receive -1 and 0.
// With a block-table row (table_row[j] = page of block j, j < nb), *page_out
// receives the selected block's table entry, unchecked (-1 where no block):
// the lookups are issued as soon as the candidates are known, so their
// latency overlaps the exact ranking. COHERENT: the scores are read with
// device-scope loads (written earlier in the same launch).
template <bool COHERENT = false>
__device__ __forceinline__ int select_blocks(const float* row, int row_len, int nb,
                                             const float (&x0)[kSelPerLane], SelectScratch& sc,
                                             int lane, float* score_out,
                                             const int32_t* table_row = nullptr,
                                             int* page_out = nullptr) {
  if (nb <= kTopK + 1) {
    const bool in = lane < nb;
    *score_out = in ? __uint_as_float(score_bits(load_score<COHERENT>(&row[min(lane, row_len - 1)])))
                    : 0.0f;
    if (table_row) *page_out = in ? table_row[min(lane, nb - 1)] : -1;
    return in ? lane : -1;
  }
  // uniform address: issued now, consumed at the end
  const int recent_page = table_row ? table_row[nb - 1] : -1;
  const int n = nb - 1;  // candidates; the recent block is always kept
  const int nchunks = (n + kSelChunk - 1) / kSelChunk;
  uint32_t v[kSelPerLane];
  // chunk c's score bits into v: chunk 0 from x0 on the first pass only, so
  // x0 is dead afterwards (later passes over several chunks reload them)
  auto chunk_bits = [&](int c, bool from_x0) {
    const int c0 = c * kSelChunk;
    float x[kSelPerLane];
    if (from_x0) {
#pragma unroll
      for (int k = 0; k < kSelPerLane; ++k) x[k] = x0[k];
    } else {
      load_score_chunk<COHERENT>(row, row_len, c0, lane, x);
    }
#pragma unroll
    for (int k = 0; k < kSelPerLane; ++k) v[k] = c0 + lane + 64 * k < n ? score_bits(x[k]) : 0u;
  };
  auto stage_chunk = [&]() {
#pragma unroll
    for (int k = 0; k < kSelPerLane; ++k) sc.stage[64 * k + lane] = v[k];
  };
  int cnt = 0;  // uniform
  if (n <= 64) {
    // at most 64 candidates: each sits in its own lane (chunk 0, k = 0), so
    // all of them go to the exact ranking below, with no threshold and no
    // compaction (the same winners: the threshold only drops non-winners)
    chunk_bits(0, true);
    if (lane < n) sc.cand[lane] = make_key(v[0], lane);
    cnt = n;
    wave_lds_sync();
  } else {
    // 1. lane maxima
    uint32_t m = 0;
    chunk_bits(0, true);
    for (int c = 0; c < nchunks; ++c) {
      if (c > 0) chunk_bits(c, false);
#pragma unroll
      for (int k = 0; k < kSelPerLane; ++k) m = max(m, v[k]);
    }
    // 2. theta: the 16th largest of the 64 lane maxima, counted with
    //    multiplicity, truncated below bit 11, by a radix select on the bit
    //    patterns: the largest x with at least 16 lanes holding a maximum >= x,
    //    decided two bits at a time from the top with three independent
    //    wavefront votes and population counts (no LDS). Score bits are
    //    non-negative, so bit 31 is clear. The truncation only admits the
    //    few candidates within ~2^-11 (relative) below the 16th largest; the
    //    exact ranking below sorts them out.
    const uint32_t theta = select_theta(m);
    // 3. compact the candidates reaching theta: a per-lane bit mask of hits,
    //    positions from a prefix sum of its population count, hit values read
    //    back from the LDS copy of the chunk (hits are rare: a lane has 0..2)
    for (int c = 0; c < nchunks; ++c) {
      const int c0 = c * kSelChunk;
      if (nchunks > 1) {
        chunk_bits(c, false);
        stage_chunk();
      } else if (c == 0) {
        stage_chunk();
      }
      uint32_t hits = 0;
#pragma unroll
      for (int k = 0; k < kSelPerLane; ++k)
        hits |= (c0 + lane + 64 * k < n && v[k] >= theta) ? (1u << k) : 0u;
      const int mine = __popc(hits);
      const int incl = wave_inclusive_sum(mine, lane);
      int pos = cnt + incl - mine;
      wave_lds_sync();
      while (hits) {
        const int k = __builtin_ctz(hits);
        hits &= hits - 1;
        if (pos < 64) sc.cand[pos] = make_key(sc.stage[64 * k + lane], c0 + lane + 64 * k);
        ++pos;
      }
      cnt += __builtin_amdgcn_readlane(incl, 63);
      wave_lds_sync();
    }
  }
  if (cnt <= 64) {
    // rank by counting against broadcast LDS reads of the candidates; the
    // candidates' pages are in flight meanwhile
    const uint64_t key = lane < cnt ? sc.cand[lane] : 0ull;
    const int cpage = (table_row && lane < cnt) ? table_row[key_block_id(key)] : -1;
    int r = 0;
    for (int s = 0; s < cnt; ++s) r += sc.cand[s] > key ? 1 : 0;
    const bool won = lane < cnt && r < kTopK;
    if (won) sc.win[r] = key;
    wave_lds_sync();
    // 4. each winner finds its place in ascending block order and writes its
    //    block, score and page there (the page is waited for only now)
    if (won) {
      const int id = key_block_id(key);
      int order = 0;
#pragma unroll
      for (int i = 0; i < kTopK; ++i) order += key_block_id(sc.win[i]) < id ? 1 : 0;
      sc.id[order] = id;
      sc.score[order] = key_score_value(key);
      sc.page[order] = cpage;
    }
  } else {
    // many candidates reach theta (equal scores): exact arg-max rounds
    uint64_t last = ~0ull;
#pragma unroll 1
    for (int r = 0; r < kTopK; ++r) {
      uint64_t best = 0;
      for (int c = 0; c < nchunks; ++c) {
        if (nchunks > 1) chunk_bits(c, false);
        const int c0 = c * kSelChunk;
#pragma unroll
        for (int k = 0; k < kSelPerLane; ++k) {
          const int j = c0 + lane + 64 * k;
          const uint64_t key = make_key(v[k], j);
          if (j < n && key < last && key > best) best = key;
        }
      }
      best = wave_max_u64(best);
      if (lane == 0) sc.win[r] = best;
      last = best;
    }
    wave_lds_sync();
    if (lane < kTopK) {
      const uint64_t key = sc.win[lane];
      const int id = key_block_id(key);
      int order = 0;
#pragma unroll
      for (int i = 0; i < kTopK; ++i) order += key_block_id(sc.win[i]) < id ? 1 : 0;
      sc.id[order] = id;
      sc.score[order] = key_score_value(key);
      sc.page[order] = table_row ? table_row[id] : -1;
    }
  }
  wave_lds_sync();
  if (lane < kTopK) {
    *score_out = sc.score[lane];
    if (table_row) *page_out = sc.page[lane];
    return sc.id[lane];
  }
  if (table_row) *page_out = lane == kTopK ? recent_page : -1;
  if (lane == kTopK) {
    *score_out = __uint_as_float(score_bits(load_score<COHERENT>(&row[nb - 1])));
    return nb - 1;
  }
  *score_out = 0.0f;
  return -1;
}

// ---------------------------------------------------------------- by W waves
// The same selection by the W wavefronts of a workgroup together, for a row
// of one chunk (64 < nb - 1 <= 2,048 candidates): wavefront w holds entries
// 512 w + 64 k + lane, k < 8, a quarter of the chunk, so the per-entry steps
// (score bits, lane maxima, hit masks, compaction) cost a quarter each. The
// union over the wavefronts of a lane's entries is the 32 entries that lane
// holds in select_blocks, so every wavefront computes the same theta from
// the combined lane maxima; the candidates of all quarters are compacted
// into one list and wavefront 0 ranks them exactly. More than 64
// candidates (many equal scores): wavefront 0 runs select_blocks on the
// whole chunk instead. Same result as select_blocks for the same row.
constexpr int kSelWaves = 4;
constexpr int kSelPerLaneWg = kSelPerLane / kSelWaves;  // 8 entries per lane
constexpr int kSelDirect = 64;  // at most this many candidates: ranked directly

struct __align__(16) SelectScratchWg {
  uint32_t lane_max[kSelWaves][64];
  int32_t wave_hits[kSelWaves];
  uint64_t cand[64];
  uint64_t win[kTopK];
  int32_t id[kTopK + 1];
  int32_t page[kTopK + 1];
};

// Wavefront w's quarter of a row's first chunk: lane l gets entries
// 512 w + 64 k + l (buffer loads over the row, entries past it read 0).
__device__ __forceinline__ void load_score_quarter(const float* row, int row_len, int wave, int lane,
                                                   float (&x)[kSelPerLaneWg]) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(row), 0, row_len * int(sizeof(float)), 0x00020000);
  const uint32_t off = uint32_t(wave * (kSelChunk / kSelWaves) + lane) * uint32_t(sizeof(float));
#pragma unroll
  for (int k = 0; k < kSelPerLaneWg; ++k)
    x[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         r, off, 64 * k * int(sizeof(float)), 0));
}

// Every thread of the workgroup calls it (it holds workgroup barriers), with
// the same nb. xq: this wavefront's quarter (load_score_quarter). sc and
// full: LDS scratch of the workgroup (full for the many-equal-scores case).
// Lane l <= 16 of every wavefront receives the block of selected slot l and
// its table entry (*page_out, unchecked), as select_blocks returns them.
__device__ __forceinline__ int select_blocks_wg(const float* row, int row_len, int nb,
                                                const float (&xq)[kSelPerLaneWg],
                                                SelectScratchWg& sc, SelectScratch& full,
                                                int wave, int lane, const int32_t* table_row,
                                                int* page_out) {
  const int n = nb - 1;  // candidates; the recent block is always kept
  const int base = wave * (kSelChunk / kSelWaves);
  uint32_t v[kSelPerLaneWg];
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kSelPerLaneWg; ++k) {
    v[k] = base + 64 * k + lane < n ? score_bits(xq[k]) : 0u;
    m = max(m, v[k]);
  }
  sc.lane_max[wave][lane] = m;
  __syncthreads();
  uint32_t mm = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) mm = max(mm, sc.lane_max[w][lane]);
  const uint32_t theta = select_theta(mm);
  uint32_t hits = 0;
#pragma unroll
  for (int k = 0; k < kSelPerLaneWg; ++k)
    hits |= (base + 64 * k + lane < n && v[k] >= theta) ? (1u << k) : 0u;
  const int mine = __popc(hits);
  const int incl = wave_inclusive_sum(mine, lane);
  if (lane == 63) sc.wave_hits[wave] = incl;
  __syncthreads();
  int before = 0, cnt = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = sc.wave_hits[w];
    before += w < wave ? c : 0;
    cnt += c;
  }
  cnt = __builtin_amdgcn_readfirstlane(cnt);  // uniform
  if (cnt <= kSelDirect) {
    int pos = before + incl - mine;
    while (hits) {
      const int k = __builtin_ctz(hits);
      hits &= hits - 1;
      uint32_t bits = v[0];
#pragma unroll
      for (int i = 1; i < kSelPerLaneWg; ++i) bits = k == i ? v[i] : bits;
      sc.cand[pos++] = make_key(bits, base + 64 * k + lane);
    }
  }
  __syncthreads();
  if (wave == 0) {
    if (cnt <= kSelDirect) {
      // rank by counting against the other candidates, read from their
      // lanes; the candidates' pages are in flight meanwhile
      const uint64_t key = lane < cnt ? sc.cand[lane] : 0ull;
      const int cpage = (table_row && lane < cnt) ? table_row[key_block_id(key)] : -1;
      const uint32_t klo = uint32_t(key), khi = uint32_t(key >> 32);
      int r = 0;
      for (int s = 0; s < cnt; ++s) {
        const uint64_t o = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(khi), s))) << 32) |
                           uint32_t(__builtin_amdgcn_readlane(int(klo), s));
        r += o > key ? 1 : 0;
      }
      const bool won = lane < cnt && r < kTopK;
      if (won) sc.win[r] = key;
      wave_lds_sync();
      // each winner finds its place in ascending block order
      if (won) {
        const int id = key_block_id(key);
        int order = 0;
#pragma unroll
        for (int i = 0; i < kTopK; ++i) order += key_block_id(sc.win[i]) < id ? 1 : 0;
        sc.id[order] = id;
        sc.page[order] = cpage;
      }
      if (lane == kTopK) {
        sc.id[kTopK] = nb - 1;
        sc.page[kTopK] = table_row ? table_row[nb - 1] : -1;
      }
    } else {
      float x0[kSelPerLane];
      load_score_chunk(row, row_len, 0, lane, x0);
      float score;
      int page = -1;
      const int id = select_blocks(row, row_len, nb, x0, full, lane, &score, table_row, &page);
      if (lane <= kTopK) {
        sc.id[lane] = id;
        sc.page[lane] = page;
      }
    }
  }
  __syncthreads();
  *page_out = lane <= kTopK ? sc.page[lane] : -1;
  return lane <= kTopK ? sc.id[lane] : -1;
}

}  // namespace msa
