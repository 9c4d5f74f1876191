/*
 * msa_nvfp4.h -- C ABI of libmsa_nvfp4.so: MiniMax-style sparse-attention
 * decode over an NVFP4 paged KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages this follows):
 *  - The KV cache and the indexer's key cache are stored as NVFP4: every 16
 *    consecutive channels of one token and one head share one E4M3 scale and
 *    hold 4-bit E2M1 codes (vLLM Delivers Day-0 Support for MiniMax M3.1
 *    Flash, section "NVFP4 KV Cache and MoE Weights"; MiniMax-M3.1-Flash lands
 *    in vLLM on day one, first paragraph: 34,560 instead of 61,440 bytes per
 *    token).
 *  - Queries stay FP8 (E4M3), so the cache is converted to FP8 before every
 *    product (same page, third paragraph). On CDNA4 the conversion is a small
 *    lookup table of scaled values plus sign handling (MiniMax-M3.1-Flash
 *    serving summary, yuxiaoba.github.io, section "AMD uses different
 *    conversion and communication mechanisms").
 *  - KV is organised in 128-token blocks; a lightweight indexer scores the
 *    context, keeps the 16 best blocks and the most recent one, and exact
 *    attention runs over those roughly 2,048 keys (same summary, section
 *    "Sparse attention still scans an index").
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is DEVICE memory owned by the caller, except the
 *    msa_pool_desc pointers, which are host memory read during the call.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream); an entry point enqueues one or two kernels on it. The library
 *    allocates nothing and, apart from the device array behind
 *    msa_indexer_decode_noalloc, keeps no state between calls; two calls may
 *    run concurrently only if they use different workspaces.
 *  - Arguments are checked on the host before anything is launched; a failed
 *    check returns a status and launches nothing. MSA_ERR_HIP reports a failed
 *    kernel launch. Device data (block tables, sequence lengths, selected ids,
 *    slots) is checked on the device: out-of-range values are never
 *    dereferenced (see each entry point for what they produce instead).
 *  - Device buffers read or written in 16-byte units must be 16-byte aligned:
 *    codes, scales, queries, workspaces, outputs.
 *  - Supported shapes: head_dim 128, block_tokens 128, topk 16, and 8 query
 *    heads per KV / index-key head (num_q_heads == 8 * num_heads); other
 *    values return MSA_ERR_UNSUPPORTED. The GQA ratio is fixed at 8 because
 *    the 8 query heads of a KV / index-key head fill half of a 16-row FP8
 *    matrix-core tile (two query tokens fill all of it in the scan): the
 *    tiles, the head-pair exchange of the scan and the attention's softmax
 *    rows are laid out for exactly 8 heads. (A general integer ratio would
 *    need other tile shapes; the workloads this library serves use 32 query
 *    heads over 4 KV heads.)
 *
 * Paged pool layout (one pool per cache: K, V and index keys), per page of
 * 128 token slots; a token in slot s lives in page s / 128, row s % 128:
 *   codes  uint8 [num_pages][num_heads][128 rows][64]  two E2M1 codes per byte,
 *          channel 2j in the low nibble of byte j, 2j+1 in the high nibble;
 *          code = sign << 3 | magnitude index (0, .5, 1, 1.5, 2, 3, 4, 6)
 *   scales uint8 [num_pages][num_heads][1024]  E4M3 scale of row r, channels
 *          16g .. 16g+15 (g = 0..7) at byte ((g/2)*16 + r%16)*16 + (r/16)*2 + g%2
 *          of its (page, head): tile-major, so one 16-byte load gives a
 *          lane all 8 row-tiles' scales of its rows and 32-channel slice.
 *          (The same bytes as a row-major [128][8] array per (page, head),
 *          permuted: a row-major array would need 8 scattered 2-byte loads
 *          per lane per block instead of one 16-byte load.)
 *
 * Sequences: sequence b has seq_lens[b] tokens in its pages, including its
 * q_per_seq query tokens (their keys are already written). Query token i of
 * sequence b (row b * q_per_seq + i of every per-query array) sits at
 * position pos = seq_lens[b] - q_per_seq + i and sees tokens 0..pos.
 * block_table[b * max_blocks + j] is the physical page of its logical block j.
 */
#ifndef MSA_NVFP4_H
#define MSA_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_HEAD_DIM 128
#define MSA_BLOCK_TOKENS 128
#define MSA_GROUP 16
#define MSA_TOPK 16
#define MSA_HEADS_PER_KV 8
#define MSA_MAX_Q_PER_SEQ 8
#define MSA_MAX_HEADS 8

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null pointer, negative size, misalignment */
  MSA_ERR_UNSUPPORTED = 2, /* a shape the library does not implement */
  MSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MSA_ERR_HIP = 4          /* the HIP runtime refused a launch */
} msa_status;

/* Shape of one paged pool. */
typedef struct msa_pool_desc {
  int32_t num_heads;    /* heads per token: KV heads, or index-key heads; 1..8 */
  int32_t head_dim;     /* channels per head; must be 128 */
  int32_t block_tokens; /* token slots per page; must be 128 */
  int32_t reserved;     /* set to 0 */
  int64_t num_pages;    /* pages in the pool; > 0 */
} msa_pool_desc;

/* Human-readable name of a status code (static storage); any other value
 * (the argument is a plain int, so no value is out of range) gives
 * "unknown msa_status". */
const char* msa_status_string(int32_t status);

/*
 * Cache writer: quantise fp32 rows to NVFP4 and store them into a pool.
 * Defines: the NVFP4 encoding above. For each (token, head, group of 16):
 *   amax = max |x|; s = E4M3 value nearest to amax/6 (ties to even,
 *   saturating at 448); each element's magnitude is the E2M1 value nearest to
 *   |x|/s (ties to even, saturating at 6; 0 when s == 0); the sign bit is
 *   kept, also for elements that round to 0.
 *   src          float [num_tokens][pool->num_heads][128]
 *   slot_mapping int64 [num_tokens]; token t goes to slot slot_mapping[t];
 *                slots < 0 or >= num_pages * 128 are skipped (not written)
 *   codes/scales the pool (layout above)
 * num_tokens == 0 is a no-op. Inputs must be finite.
 */
msa_status msa_nvfp4_quantize(const msa_pool_desc* pool, const float* src,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              uint8_t* codes, uint8_t* scales, void* stream);

/*
 * Workspace bytes msa_indexer_decode needs: the fp32 block scores
 * [num_seqs * q_per_seq][max_blocks]. No initial contents are required.
 */
size_t msa_indexer_workspace_bytes(int32_t num_seqs, int32_t q_per_seq, int32_t max_blocks);

/*
 * Indexer: scan the whole NVFP4 index-key cache of every sequence, score its
 * 128-token blocks against FP8 index queries and select, per query token,
 * the 16 best blocks plus the most recent one.
 * Defines (the build's reading of "a lightweight indexer scores context"):
 *   S(t)  = sum_h w_h * max(0, q_h . K(t, h / 8)), K = the FP8 dequantised key
 *   B(j)  = max of S(t) over the visible tokens of block j
 *   ids   = top-16 of blocks 0..nb-2 by (B descending, j ascending), plus block
 *           nb-1, in ascending order; all blocks when nb <= 17; -1 padding.
 *           nb = pos / 128 + 1.
 *   idx          pool of index keys (num_heads = index-key heads)
 *   q_fp8        uint8 E4M3 [num_seqs * q_per_seq][num_q_heads][128]
 *   head_w       float [num_seqs * q_per_seq][num_q_heads]; must be >= 0
 *   block_table  int32 [num_seqs][max_blocks]
 *   seq_lens     int32 [num_seqs]
 *   out_ids      int32 [num_seqs * q_per_seq][topk + 1]
 *   out_scores   float [num_seqs * q_per_seq][topk + 1] or NULL: B(j) of each
 *                selected block (0 for padding)
 * Device-side checks: a sequence with seq_lens < q_per_seq or
 * seq_lens > max_blocks * 128 gets all ids -1; a block whose page id is
 * outside [0, num_pages) scores 0 and its page is not read.
 * 1 <= q_per_seq <= 8; topk must be 16.
 */
msa_status msa_indexer_decode(const msa_pool_desc* idx, const uint8_t* idx_codes,
                              const uint8_t* idx_scales, const uint8_t* q_fp8,
                              const float* head_w, int32_t num_q_heads,
                              const int32_t* block_table, int32_t max_blocks,
                              const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                              int32_t topk, int32_t* out_ids, float* out_scores,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_indexer_decode for callers that cannot allocate device memory or pass
 * a workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. The same arguments without the workspace, and the
 * same results: the block scores live in a device array of the library
 * (MSA_NOALLOC_MAX_SCORES fp32 values, 4 MiB, one copy per GPU, held until the
 * process ends) instead of the caller's workspace.
 *   num_seqs * q_per_seq * max_blocks must not exceed MSA_NOALLOC_MAX_SCORES
 *   (else MSA_ERR_WORKSPACE, nothing launched).
 * The first call on a device looks the array's address up (no allocation);
 * every call on one GPU shares the array, so calls that may overlap on one
 * GPU (other streams, other threads) race on it and must be serialised by
 * the caller. Its contents need no initialisation: each call writes every
 * score it reads. Other arguments, device-side checks and errors as
 * msa_indexer_decode.
 */
#define MSA_NOALLOC_MAX_SCORES (1 << 20)
msa_status msa_indexer_decode_noalloc(const msa_pool_desc* idx, const uint8_t* idx_codes,
                                      const uint8_t* idx_scales, const uint8_t* q_fp8,
                                      const float* head_w, int32_t num_q_heads,
                                      const int32_t* block_table, int32_t max_blocks,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t q_per_seq, int32_t topk, int32_t* out_ids,
                                      float* out_scores, void* stream);

/*
 * The indexer in two stages, for callers that keep the block scores (for
 * example to merge candidates gathered from several context shards).
 * msa_indexer_decode is exactly msa_indexer_scan followed by
 * msa_indexer_select on its workspace.
 *
 * msa_indexer_scan writes B(j) for every visible block j < nb of every
 * query token into block_scores float [num_seqs * q_per_seq][max_blocks];
 * entries past a query token's nb are left untouched. Same arguments and
 * device-side checks as msa_indexer_decode.
 */
msa_status msa_indexer_scan(const msa_pool_desc* idx, const uint8_t* idx_codes,
                            const uint8_t* idx_scales, const uint8_t* q_fp8, const float* head_w,
                            int32_t num_q_heads, const int32_t* block_table, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                            float* block_scores, void* stream);

/*
 * msa_indexer_scan for a batch in which groups of sequences share leading
 * blocks: the same physical pages at the same logical block indices, as a
 * cached common prefix gives (MiniMax-M3.1-Flash serving summary, section
 * "AMD uses different conversion and communication mechanisms": shared
 * prefixes reduce repeated dequantisation across requests). One launch: each
 * shared block is read once and dequantised once, into registers, and scored
 * against the query tokens of every member of its group; the other blocks
 * are scanned as by msa_indexer_scan, by the same kernel. The block scores
 * are the values msa_indexer_scan writes for the same inputs.
 * Groups (device arrays; msa_shared_prefix_groups derives them from a host
 * copy of the block table):
 *   num_groups         0 .. 65535 (0: msa_indexer_scan)
 *   group_lead         int32 [num_groups]: a sequence whose pages define the
 *                      group's shared pages
 *   group_blocks       int32 [num_groups]: leading blocks the group shares
 *   max_group_blocks   host: >= every group_blocks entry, in [1, max_blocks]
 *                      (ignored when num_groups == 0)
 *   seq_group          int32 [num_seqs]: the group of each sequence, -1: none
 * Block j of sequence b is scored by its group's shared pass when
 * g = seq_group[b] is in [0, num_groups), j < min(group_blocks[g],
 * max_blocks), group_lead[g] is a sequence of the batch, and b's page of
 * block j equals the lead's; otherwise by the regular scan. Any group arrays
 * therefore give the scores of msa_indexer_scan; groups that do not match
 * the block table only share less. Other arguments as msa_indexer_scan.
 */
msa_status msa_indexer_scan_shared(const msa_pool_desc* idx, const uint8_t* idx_codes,
                                   const uint8_t* idx_scales, const uint8_t* q_fp8,
                                   const float* head_w, int32_t num_q_heads,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                                   int32_t num_groups, const int32_t* group_lead,
                                   const int32_t* group_blocks, int32_t max_group_blocks,
                                   const int32_t* seq_group, float* block_scores, void* stream);

/*
 * Shared-prefix groups of a batch, derived on the host from a HOST copy of
 * its block table and sequence lengths (a serving engine keeps both): the
 * sequences with a valid length (q_per_seq <= seq_lens[b] <= max_blocks * 128)
 * are grouped by the page of their block 0; a group of two or more members
 * shares the longest run of leading blocks whose pages are the same, and
 * not negative, in every member, within every member's own blocks
 * (ceil(seq_lens / 128)); its lead is its lowest-numbered member. Groups are
 * numbered in the order of their leads.
 *   block_table int32 [num_seqs][max_blocks], seq_lens int32 [num_seqs]: host
 *   group_lead, group_blocks: host int32 arrays of num_seqs entries (the first
 *               *num_groups are written); seq_group: host int32 [num_seqs]
 *               (-1 for a sequence in no group)
 *   *num_groups, *max_group_blocks: host outputs (0, 0 with no group)
 * The outputs, copied to the device, are msa_indexer_scan_shared's group
 * arguments. Runs on the calling thread; no device work.
 */
msa_status msa_shared_prefix_groups(const int32_t* block_table, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                                    int32_t* group_lead, int32_t* group_blocks, int32_t* seq_group,
                                    int32_t* num_groups, int32_t* max_group_blocks);

/*
 * msa_indexer_select reads block_scores (as written by msa_indexer_scan) and
 * writes out_ids / out_scores exactly as msa_indexer_decode does; scores
 * must be finite (negative values and -0 rank as 0).
 */
msa_status msa_indexer_select(const float* block_scores, const int32_t* seq_lens,
                              int32_t max_blocks, int32_t num_seqs, int32_t q_per_seq,
                              int32_t topk, int32_t* out_ids, float* out_scores, void* stream);

/*
 * Cache insertion after the QKV projection, in one launch: the pages'
 * fused projection / normalisation / RoPE / cache-insertion path, which
 * avoids writing the intermediate tensor to HBM and reading it back
 * (MiniMax-M3.1-Flash serving summary, section "Reduce both data movement
 * and resource waits"); the projection itself is the caller's. Per token t:
 *   1. optional RMSNorm of every query head (q and q_idx, weight q_norm_w)
 *      and key head (k and k_idx, weight k_norm_w):
 *      y = x / sqrt(mean(x^2) + rms_eps) * w; V is not normalised;
 *   2. RoPE, rotate-half form, on channels 0 .. rotary_dim-1 of the q, q_idx,
 *      k and k_idx heads: for i < rotary_dim/2 the pair (i, i + rotary_dim/2)
 *      is rotated by positions[t] * rope_theta^(-2i/rotary_dim) radians;
 *   3. k, v and k_idx are encoded to NVFP4 exactly as msa_nvfp4_quantize
 *      would encode the fp32 values, into slot slot_mapping[t] of their pools
 *      (slots < 0 or past the pool: not stored);
 *   4. q and q_idx are rounded to FP8 E4M3 (nearest even, clamped to +-448).
 * Arithmetic is fp32 (the angles are evaluated in fp64).
 *   qkv          bf16 bit patterns [num_tokens][(8 Hkv + 8 Hidx + 2 Hkv +
 *                Hidx) * 128]: heads q (8 Hkv), q_idx (8 Hidx), k (Hkv),
 *                v (Hkv), k_idx (Hidx), Hkv = kv->num_heads,
 *                Hidx = idx->num_heads; 16-byte aligned
 *   positions    int32 [num_tokens]; slot_mapping int64 [num_tokens]
 *   kv, idx      shapes of the K / V pools and of the index-key pool
 *   q_norm_w, k_norm_w  float [128] or NULL (no normalisation)
 *   rotary_dim   0, 32, 64, 96 or 128 (else MSA_ERR_UNSUPPORTED); rope_theta
 *                > 1 when rotary_dim > 0
 *   q_fp8        uint8 [num_tokens][8 Hkv][128]; q_idx_fp8 uint8
 *                [num_tokens][8 Hidx][128]
 * One kernel on `stream`; no workspace.
 */
msa_status msa_qkv_rope_insert(const uint16_t* qkv, int64_t num_tokens, const int32_t* positions,
                               const int64_t* slot_mapping, const msa_pool_desc* kv,
                               uint8_t* k_codes, uint8_t* k_scales, uint8_t* v_codes,
                               uint8_t* v_scales, const msa_pool_desc* idx, uint8_t* idx_codes,
                               uint8_t* idx_scales, const float* q_norm_w, const float* k_norm_w,
                               float rms_eps, int32_t rotary_dim, float rope_theta,
                               uint8_t* q_fp8, uint8_t* q_idx_fp8, void* stream);

/*
 * Workspace bytes msa_sparse_attn_decode needs for its split partial results
 * (running max, denominator and unnormalised output per split) and, after
 * them, one arrival counter per (query token, KV head) pair: the pair's last
 * split to finish merges the partials. 0 when the launch plan has one split
 * per pair. Zero-fill a workspace once before its first use; every call
 * leaves the counters zero again, so later calls need no refill (a call
 * that does not run to completion, or two overlapping calls on one
 * workspace, void this).
 */
size_t msa_attn_workspace_bytes(int32_t num_seqs, int32_t q_per_seq, int32_t num_q_heads,
                                int32_t num_sel);

/*
 * Sparse attention: for each query token and query head h, exact softmax
 * attention over the visible tokens (t <= pos) of the selected blocks,
 *   o = sum_t softmax_t(softmax_scale * q_h . K(t)) V(t),  KV head h / 8,
 * with K and V dequantised to FP8 from their NVFP4 pools.
 *   kv           shape of both pools (num_heads = KV heads)
 *   q_fp8        uint8 E4M3 [num_seqs * q_per_seq][num_q_heads][128]
 *   sel_ids      int32 [num_seqs * q_per_seq][num_sel] logical block ids,
 *                distinct; entries < 0, >= max_blocks, past pos, or whose
 *                page is outside [0, num_pages) are ignored
 *   out          float [num_seqs * q_per_seq][num_q_heads][128]; a query
 *                token with no usable block gets zeros
 *   workspace    msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads,
 *                num_sel) bytes, 256-byte aligned, zero-filled before its
 *                first use (MSA_ERR_WORKSPACE if smaller or misaligned)
 * 1 <= num_sel <= 64. The softmax weights enter the P x V product as two
 * FP8 terms, FP8(256 p) + FP8(16 (256 p - FP8(256 p))) / 16 (about 8
 * significant bits); the denominator sums the same rounded terms.
 */
msa_status msa_sparse_attn_decode(const msa_pool_desc* kv, const uint8_t* k_codes,
                                  const uint8_t* k_scales, const uint8_t* v_codes,
                                  const uint8_t* v_scales, const uint8_t* q_fp8,
                                  int32_t num_q_heads, const int32_t* block_table,
                                  int32_t max_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t q_per_seq, const int32_t* sel_ids, int32_t num_sel,
                                  float softmax_scale, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Selection and sparse attention in one launch: the blocks of each query
 * token are selected from block_scores (as written by msa_indexer_scan)
 * inside the attention kernel, then attended as by msa_sparse_attn_decode.
 * For the same block scores the result equals msa_indexer_select followed by
 * msa_sparse_attn_decode with num_sel = topk + 1: the same ids and the same
 * output bits. It saves the selection kernel's launch and the round trip of
 * the ids through memory at low concurrency (the pages' mono-kernel for small
 * batches: MiniMax-M3.1-Flash serving summary, section "AMD uses different
 * conversion and communication mechanisms").
 *   block_scores float [num_seqs * q_per_seq][max_blocks]; finite
 *   topk         must be 16
 *   out_ids      int32 [num_seqs * q_per_seq][topk + 1] or NULL: the
 *                selected ids, as msa_indexer_select writes them
 *   workspace    msa_attn_workspace_bytes(num_seqs, q_per_seq, num_q_heads,
 *                topk + 1) bytes, zero-filled before its first use
 * Other arguments and device-side checks as msa_sparse_attn_decode; a
 * sequence with seq_lens < q_per_seq or seq_lens > max_blocks * 128 gets ids
 * -1 and zero output.
 */
msa_status msa_sparse_attn_select_decode(const msa_pool_desc* kv, const uint8_t* k_codes,
                                         const uint8_t* k_scales, const uint8_t* v_codes,
                                         const uint8_t* v_scales, const uint8_t* q_fp8,
                                         int32_t num_q_heads, const int32_t* block_table,
                                         int32_t max_blocks, const int32_t* seq_lens,
                                         int32_t num_seqs, int32_t q_per_seq,
                                         const float* block_scores, int32_t topk,
                                         int32_t* out_ids, float softmax_scale, float* out,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes msa_decode_mono needs: the fp32 block scores
 * [num_seqs * q_per_seq][max_blocks] (at offset 0), the attention partials of
 * every block, and the launch's arrival counters. Zero-fill it before its
 * first use: the counters must start at zero, and a call leaves them zero as
 * long as none of its bounded waits times out (the error word, below, stays
 * 0). After a timeout the counters may hold late arrivals: zero the counter
 * region again (the caller's, once the stream is idle) before reusing the
 * workspace.
 */
size_t msa_decode_mono_workspace_bytes(int32_t num_seqs, int32_t q_per_seq, int32_t num_q_heads,
                                       int32_t max_blocks);

/*
 * The whole decode step in one kernel launch, for low concurrency: the index
 * scan of msa_indexer_scan, the selection and the attention of
 * msa_sparse_attn_select_decode, with the same ids and the same output bits
 * as those two calls make when the attention runs one workgroup per selected
 * block (num_seqs * q_per_seq * 4 KV heads * 17 <= 384). The pages keep a
 * separate mono-kernel strategy for low concurrency to reduce launches, and
 * note that one kernel arrangement need not suit every regime
 * (MiniMax-M3.1-Flash serving summary, sections "AMD uses different
 * conversion and communication mechanisms" and "Keep capacity, layer, and
 * system results separate").
 * How: the attention partial (m, l, o) of EVERY block of every query token
 * and KV head is computed while the scan runs, and per (query token, KV head)
 * a last workgroup waits for both, selects the 16 + 1 blocks from the scores
 * and merges only their partials. That costs max_blocks x 73,728 bytes of K/V
 * reads per sequence instead of 17 x 73,728, so the launch is bounded to the
 * shapes where that costs less than the launches it saves:
 * num_seqs * q_per_seq * 4 * max_blocks <= 1024, e.g. 1 x 32K, 2 x 16K,
 * 8 x 4K tokens with one query token (else MSA_ERR_UNSUPPORTED).
 *   idx, idx_codes, idx_scales, q_idx_fp8, head_w   as msa_indexer_scan; the
 *                index pool must have 4 heads
 *   kv, k_*, v_*, q_fp8, num_q_heads, block_table, max_blocks, seq_lens,
 *   num_seqs, q_per_seq, softmax_scale, out   as msa_sparse_attn_decode; the
 *                KV pools must have 4 heads (num_q_heads = 32); the index and
 *                KV pools share the block table
 *   topk         must be 16
 *   out_ids      int32 [num_seqs * q_per_seq][17] or NULL: the selected ids,
 *                as msa_indexer_select writes them
 *   workspace    msa_decode_mono_workspace_bytes(...) bytes, 256-byte aligned,
 *                zero-filled before its first use (see above); it must not be
 *                shared by calls that may overlap
 * Device-side checks as msa_sparse_attn_select_decode. The launch's
 * workgroups wait only for workgroups dispatched before them; each wait is
 * still bounded (20 ms), and one that times out gives that query token zero
 * output and ids -1 and sets the error word, the last 32-bit word of the
 * msa_decode_mono_workspace_bytes(...) bytes, to 1; it stays set until the
 * caller zeroes it. The counter region is the last
 * align256(4 * ((num_seqs + pairs) * 128 + num_seqs * 16 + 1)) bytes of
 * those, pairs = num_seqs * q_per_seq * 4.
 */
msa_status msa_decode_mono(const msa_pool_desc* idx, const uint8_t* idx_codes,
                           const uint8_t* idx_scales, const uint8_t* q_idx_fp8,
                           const float* head_w, const msa_pool_desc* kv, const uint8_t* k_codes,
                           const uint8_t* k_scales, const uint8_t* v_codes,
                           const uint8_t* v_scales, const uint8_t* q_fp8, int32_t num_q_heads,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t q_per_seq,
                           int32_t topk, int32_t* out_ids, float softmax_scale, float* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement: a plain streaming read of `bytes` bytes at `buf`, the read
 * ceiling a bandwidth-bound kernel of this library is compared with (the
 * index scan streams the whole index cache once per step: MiniMax-M3.1-Flash
 * serving summary, section "Sparse attention still scans an index"). Each
 * workgroup reads one contiguous chunk of chunk_bytes with the index scan's
 * loads (16-byte non-temporal, 8 in flight per lane) and folds them with
 * XOR; sink (uint32 [ceil(bytes / chunk_bytes)], device) is written only if
 * a fold hits a fixed pattern, so the traffic is the buffer's bytes.
 * buf 16-byte aligned; bytes and chunk_bytes multiples of 16, chunk_bytes in
 * (0, 2^30]. One kernel on `stream`.
 */
msa_status msa_read_probe(const void* buf, int64_t bytes, int64_t chunk_bytes, uint32_t* sink,
                          void* stream);

/*
 * Measurement: plain streaming reads and writes at once, the ceiling of a
 * kernel with a given read:write mix (the cache writer reads the projection
 * rows and writes the cache rows and FP8 queries: MiniMax-M3.1-Flash serving
 * summary, section "Reduce both data movement and resource waits").
 * Workgroup i reads chunk_bytes of src from byte i * chunk_bytes (the
 * read probe's loads) and writes ceil(write_bytes / grid) bytes of dst
 * (rounded up to 16) from byte i times that, in 32 KiB steps spread evenly
 * over its reads (the last with its last read), with 16-byte non-temporal
 * stores of read words XOR the fold of the words read so far (every load
 * feeds a store); grid = ceil(read_bytes / chunk_bytes). Nothing outside
 * [src, src + read_bytes) and [dst, dst + write_bytes) is touched; with
 * write_bytes 0 nothing is read either.
 * src and dst 16-byte aligned (dst may be null when write_bytes is 0);
 * read_bytes > 0 (or both 0: nothing is launched), write_bytes and
 * chunk_bytes multiples of 16, chunk_bytes in (0, 2^30]. One kernel on
 * `stream`.
 */
msa_status msa_stream_probe(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                            int64_t chunk_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_NVFP4_H */
