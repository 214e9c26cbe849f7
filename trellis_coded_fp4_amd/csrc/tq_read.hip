// tq_read.hip -- a plain streaming-read kernel: the practical read rate of
// HBM at a given size, measured beside the layer kernels (the layer's
// compressed bytes are read once per call, so this is the ceiling its
// GB/s is compared with).
//
// Each thread reads four 16-byte vectors per pass, all in flight before
// any is used, grid-stride over the buffer (four workgroups per compute
// unit); the XOR of every 32-bit word is folded into one word per
// workgroup, and each workgroup XORs it atomically into one of the 256
// sink words (workgroup index mod 256, so the atomics do not queue on one
// address). The XOR of the 256 sink words is the checksum.
#include <hip/hip_runtime.h>

#include "trellis.h"

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;   // 16-byte loads in flight per thread and pass
constexpr int kSink = 256;  // sink words

__global__ void __launch_bounds__(kThreads) k_read(const uint4 *p, size_t n16, const uint32_t *tail, size_t n4tail,
                                                   uint32_t *sink) {
  uint32_t x = 0;
  const size_t stride = (size_t)gridDim.x * kThreads * kVec;
  for (size_t i = (size_t)blockIdx.x * kThreads * kVec + threadIdx.x; i < n16; i += stride) {
    uint4 v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const size_t k = i + (size_t)j * kThreads;
      v[j] = k < n16 ? p[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  // the bytes past the last whole 16-byte vector (fewer than four words)
  if (blockIdx.x == 0 && threadIdx.x < n4tail) x ^= tail[threadIdx.x];
  // wave XOR, the waves' words through LDS, one atomic per workgroup
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) v ^= part[i];
    atomicXor(sink + (blockIdx.x & (kSink - 1)), v);
  }
}

}  // namespace

extern "C" int trellis_read_bandwidth(hipStream_t stream, const void *buf, size_t bytes, uint32_t *sink) {
  if (!buf || !sink) return TRELLIS_ENULL;
  if (((uintptr_t)buf & 15) || (bytes & 3)) return TRELLIS_EINVAL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return TRELLIS_EHIP;
  const size_t n16 = bytes / 16, n4tail = (bytes % 16) / 4;
  const size_t per_block = (size_t)kThreads * kVec;
  const size_t want = (n16 + per_block - 1) / per_block;
  const int blocks = (int)(want < 1 ? 1 : (want > (size_t)cus * 4 ? (size_t)cus * 4 : want));
  hipLaunchKernelGGL(k_read, dim3(blocks), dim3(kThreads), 0, stream, (const uint4 *)buf, n16,
                     (const uint32_t *)buf + 4 * n16, n4tail, sink);
  return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_EHIP;
}
