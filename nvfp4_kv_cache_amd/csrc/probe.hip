// probe.hip -- msa_read_probe: a plain streaming read of a device buffer,
// the ceiling a bandwidth-bound kernel of this library is compared with.
// Each workgroup reads one contiguous chunk with the loads the index scan
// uses (16-byte non-temporal buffer loads, 8 in flight per lane) and folds
// the bytes with XOR; nothing is written unless the fold hits a fixed
// pattern, so the traffic is the buffer's bytes and the workgroups' sink
// words at most.
#include "msa_nvfp4.h"
#include "nvfp4_tile.h"
#include "scan_body.h"

namespace msa {

constexpr int kProbeThreads = 256;
constexpr int kProbeInFlight = 8;
constexpr uint32_t kProbePattern = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t* buf,
                                                                   int64_t bytes, int64_t chunk,
                                                                   uint32_t* sink) {
  const int64_t begin = int64_t(blockIdx.x) * chunk;
  const int64_t n = min(chunk, bytes - begin);  // > 0 by the grid
  // one buffer descriptor per workgroup over its chunk (at most 2 GiB):
  // loads past the chunk return zeros and read nothing
  const auto r = tile_rsrc(buf + begin, int(n));
  // every offset is in the lane (vector) offset, which the range check covers
  const uint32_t lane_off = threadIdx.x * 16u;
  constexpr uint32_t kStep = kProbeThreads * 16;
  uint32_t acc = 0;
  for (int64_t off = 0; off < n; off += int64_t(kStep) * kProbeInFlight) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k)
      v[k] = load_tile16(r, lane_off + uint32_t(off) + k * kStep, 0);
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  if (acc == kProbePattern) sink[blockIdx.x] = acc;
}

}  // namespace msa

extern "C" msa_status msa_read_probe(const void* buf, int64_t bytes, int64_t chunk_bytes,
                                     uint32_t* sink, void* stream) {
  using namespace msa;
  if (bytes < 0 || chunk_bytes <= 0) return MSA_ERR_INVALID_ARG;
  if (bytes == 0) return MSA_OK;
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || (bytes & 15) ||
      (chunk_bytes & 15) || chunk_bytes > (int64_t(1) << 30))
    return MSA_ERR_INVALID_ARG;
  const int64_t grid = (bytes + chunk_bytes - 1) / chunk_bytes;
  if (grid > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(grid)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(buf), bytes,
                     chunk_bytes, sink);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
