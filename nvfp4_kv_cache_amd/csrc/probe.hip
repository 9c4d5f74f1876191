// probe.hip -- plain streaming kernels, the ceilings the bandwidth-bound
// kernels of this library are compared with.
// msa_read_probe: each workgroup reads one contiguous chunk of a buffer with
// the loads the index scan uses (16-byte non-temporal buffer loads, 8 in
// flight per lane) and folds the bytes with XOR; nothing is written unless
// the fold hits a fixed pattern, so the traffic is the buffer's bytes and
// the workgroups' sink words at most.
// msa_stream_probe: the same reads, with a second buffer written at the
// same time in a given proportion (the read:write mix of a cache writer).
#include "msa_nvfp4.h"
#include "nvfp4_tile.h"

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

// Workgroup i reads bytes [i rchunk, (i + 1) rchunk) of src in iterations
// of 32 KiB (8 loads of 16 bytes per lane) and writes bytes
// [i wchunk, (i + 1) wchunk) of dst in 32 KiB iterations spread evenly over
// its reads, the last one with its last read. A written word is a word of
// the current iteration XOR the fold of every word the lane has read so
// far, so every load feeds a store and none can be dropped or moved into
// the write branch. Descriptors bound both ranges: accesses past them read
// zeros and write nothing.
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(
    const uint8_t* src, int64_t rbytes, int64_t rchunk, uint8_t* dst, int64_t wbytes,
    int64_t wchunk) {
  const int64_t rb = int64_t(blockIdx.x) * rchunk, wb = int64_t(blockIdx.x) * wchunk;
  const int rn = int(min(rchunk, rbytes - rb));  // > 0 by the grid
  const int wn = int(max(int64_t(0), min(wchunk, wbytes - wb)));
  const auto r = tile_rsrc(src + rb, rn);
  const auto w = tile_rsrc(dst + min(wb, wbytes), wn);
  const uint32_t lane_off = threadIdx.x * 16u;
  constexpr int kStep = kProbeThreads * 16;
  constexpr int kIter = kStep * kProbeInFlight;
  const int nr = (rn + kIter - 1) / kIter, nw = (wn + kIter - 1) / kIter;
  int wdone = 0;
  uint32_t acc = kProbePattern;
  for (int it = 0; it < nr; ++it) {
    uint4 v[kProbeInFlight];
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k)
      v[k] = load_tile16(r, lane_off + uint32_t(it) * kIter + k * kStep, 0);
#pragma unroll
    for (int k = 0; k < kProbeInFlight; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    const int wto = int((int64_t(it) + 1) * nw / nr);
    for (; wdone < wto; ++wdone) {
#pragma unroll
      for (int k = 0; k < kProbeInFlight; ++k) {
        const auto o = __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned,
                                          make_uint4(v[k].x ^ acc, v[k].y, v[k].z, v[k].w));
        __builtin_amdgcn_raw_buffer_store_b128(o, w, lane_off + uint32_t(wdone) * kIter + k * kStep,
                                               0, kLoadNonTemporal);
      }
    }
  }
}

}  // namespace msa

extern "C" msa_status msa_stream_probe(const void* src, int64_t read_bytes, void* dst,
                                       int64_t write_bytes, int64_t chunk_bytes, void* stream) {
  using namespace msa;
  if (read_bytes < 0 || write_bytes < 0 || chunk_bytes <= 0) return MSA_ERR_INVALID_ARG;
  if (read_bytes == 0) return write_bytes == 0 ? MSA_OK : MSA_ERR_INVALID_ARG;
  if (!src || (write_bytes > 0 && !dst) || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15) || (read_bytes & 15) || (write_bytes & 15) ||
      (chunk_bytes & 15) || chunk_bytes > (int64_t(1) << 30))
    return MSA_ERR_INVALID_ARG;
  const int64_t grid = (read_bytes + chunk_bytes - 1) / chunk_bytes;
  if (grid > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  // each workgroup's share of the writes, in whole 16-byte words
  const int64_t wchunk = ((write_bytes + grid - 1) / grid + 15) / 16 * 16;
  if (wchunk > (int64_t(1) << 30)) return MSA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(stream_probe_kernel, dim3(unsigned(grid)), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(src), read_bytes,
                     chunk_bytes, static_cast<uint8_t*>(dst), write_bytes, wchunk);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

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
