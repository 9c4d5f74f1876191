// quantize.hip -- msa_nvfp4_quantize: the NVFP4 paged-cache writer.
//
// One thread per (token, head, 16-channel group): it reads the group's 64
// source bytes, picks the E4M3 scale nearest to amax/6 and the E2M1 code of
// every element, and writes 8 code bytes plus 1 scale byte into the token's
// page row. Both roundings are decided by exact fp32 comparisons: amax
// against 6 x (midpoint of two E4M3 values) and |x| against
// s x (midpoint of two E2M1 values); every such bound has at most 7
// significant bits, so no division and no rounding of the bounds occur.
// Format: NVFP4 as reproduced by the pages' 34,560 bytes per token
// (MiniMax-M3.1-Flash lands in vLLM on day one, first paragraph).
#include "msa_nvfp4.h"
#include "nvfp4_encode.h"

namespace msa {

__constant__ ScaleBounds kScaleBnd = make_scale_bounds();

__global__ __launch_bounds__(256) void nvfp4_quantize_kernel(
    const float* __restrict__ src, const int64_t* __restrict__ slot_mapping, int64_t num_groups,
    int num_heads, int64_t num_slots, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ float bnd[128];
  if (threadIdx.x < 128) bnd[threadIdx.x] = kScaleBnd.b[threadIdx.x];
  __syncthreads();

  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= num_groups) return;
  const int g = int(gid % kScaleRow);
  const int64_t th = gid / kScaleRow;  // token * num_heads + head
  const int h = int(th % num_heads);
  const int64_t t = th / num_heads;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;

  const float4* p = reinterpret_cast<const float4*>(src + gid * kGroup);
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 v = p[i];
    x[4 * i + 0] = v.x;
    x[4 * i + 1] = v.y;
    x[4 * i + 2] = v.z;
    x[4 * i + 3] = v.w;
  }
  uint32_t packed[2];
  const int sb = nvfp4_encode_group(x, bnd, packed);

  const int64_t page = slot / kBlockTokens;
  const int row = int(slot % kBlockTokens);
  const int64_t page_head = page * num_heads + h;
  *reinterpret_cast<uint2*>(codes + (page_head * kBlockTokens + row) * kCodeRow + g * 8) =
      make_uint2(packed[0], packed[1]);
  scales[page_head * kScalePage + scale_offset(row, g)] = uint8_t(sb);
}

}  // namespace msa

extern "C" msa_status msa_nvfp4_quantize(const msa_pool_desc* pool, const float* src,
                                         const int64_t* slot_mapping, int64_t num_tokens,
                                         uint8_t* codes, uint8_t* scales, void* stream) {
  if (!pool || num_tokens < 0) return MSA_ERR_INVALID_ARG;
  if (pool->head_dim != MSA_HEAD_DIM || pool->block_tokens != MSA_BLOCK_TOKENS)
    return MSA_ERR_UNSUPPORTED;
  if (pool->num_heads < 1 || pool->num_heads > MSA_MAX_HEADS) return MSA_ERR_UNSUPPORTED;
  if (pool->num_pages <= 0) return MSA_ERR_INVALID_ARG;
  if (num_tokens == 0) return MSA_OK;
  if (!src || !slot_mapping || !codes || !scales) return MSA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(codes) & 15) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7))
    return MSA_ERR_INVALID_ARG;
  const int64_t num_groups = num_tokens * pool->num_heads * msa::kScaleRow;
  const int64_t blocks = (num_groups + 255) / 256;
  if (blocks > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(msa::nvfp4_quantize_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), src, slot_mapping, num_groups,
                     pool->num_heads, pool->num_pages * MSA_BLOCK_TOKENS, codes, scales);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
