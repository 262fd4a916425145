// Read-only HBM streams: the practical bandwidth ceiling that the weight-streaming kernels are
// measured against.  A kernel that only reads shows what the memory system delivers to loads
// alone, without the write traffic of a copy and without any arithmetic.
//
// Two access patterns:
//   linear -- the buffer as one run of 16-byte vectors, grid-strided, eight loads in flight
//             per lane: the easiest pattern for the memory system;
//   tiles  -- the weight layout of the GEMM kernels: the buffer as rows of row_bytes, one wave
//             per tile of 16 consecutive rows; at step j lane l reads the 16 bytes at
//             64 j + 16 (l / 16) of row l % 16, so one load instruction takes 64 bytes from
//             each of 16 rows, and a wave walks its rows from start to end.
// Each workgroup writes the XOR of the 16-byte vectors it read to sink[blockIdx.x]: the loads
// cannot be removed, and the XOR over all entries (which equals the XOR of the buffer's
// vectors under either pattern) checks that every vector was read exactly once.
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// XOR of `v` over the workgroup, stored by thread 0 to sink[blockIdx.x].
__device__ __forceinline__ void block_xor_store(u32x4 v, u32x4* __restrict__ sink) {
  __shared__ u32x4 part[kThreads / 64];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] ^= (uint32_t)__shfl_xor((int)v[c], d, 64);
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 s = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_linear_kernel(const u32x4* __restrict__ src,
                                                               size_t nvec,
                                                               u32x4* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < nvec; i += stride) acc ^= load16<NT>(src + i);
  block_xor_store(acc, sink);
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void read_tiles_kernel(const unsigned char* __restrict__ src,
                                                              int row_bytes, int tiles,
                                                              u32x4* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;
  const int nwaves = gridDim.x * (kThreads / 64);
  const int steps = row_bytes / 64;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int t = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6); t < tiles; t += nwaves) {
    const u32x4* row = reinterpret_cast<const u32x4*>(src + ((size_t)t * 16 + r) * row_bytes) + kg;
    int j = 0;
    for (; j + kUnroll <= steps; j += kUnroll) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = load16<NT>(row + (size_t)(j + u) * 4);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; j < steps; ++j) acc ^= load16<NT>(row + (size_t)j * 4);
  }
  block_xor_store(acc, sink);
}

}  // namespace
}  // namespace qv

using namespace qv;

extern "C" qv_status_t qv_test_read_stream(const void* src, size_t bytes, int pattern,
                                           int row_bytes, int nontemporal, int blocks,
                                           uint32_t* sink, void* stream) {
  if (!src || !sink) return QV_ERR_NULL;
  if (pattern != QV_READ_LINEAR && pattern != QV_READ_TILES) return QV_ERR_SHAPE;
  if (blocks < 1 || blocks > QV_READ_MAX_BLOCKS || bytes == 0 || bytes % 16 != 0) return QV_ERR_SHAPE;
  if (((uintptr_t)src % 16) != 0 || ((uintptr_t)sink % 16) != 0) return QV_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  u32x4* out = reinterpret_cast<u32x4*>(sink);
  if (pattern == QV_READ_LINEAR) {
    const u32x4* p = static_cast<const u32x4*>(src);
    if (nontemporal) read_linear_kernel<true><<<blocks, kThreads, 0, s>>>(p, bytes / 16, out);
    else read_linear_kernel<false><<<blocks, kThreads, 0, s>>>(p, bytes / 16, out);
  } else {
    if (row_bytes < 64 || row_bytes % 64 != 0 || bytes % ((size_t)16 * row_bytes) != 0)
      return QV_ERR_SHAPE;
    const size_t tiles = bytes / ((size_t)16 * row_bytes);
    if (tiles > (size_t)INT32_MAX) return QV_ERR_SHAPE;
    const unsigned char* p = static_cast<const unsigned char*>(src);
    if (nontemporal) read_tiles_kernel<true><<<blocks, kThreads, 0, s>>>(p, row_bytes, (int)tiles, out);
    else read_tiles_kernel<false><<<blocks, kThreads, 0, s>>>(p, row_bytes, (int)tiles, out);
  }
  return hipGetLastError() == hipSuccess ? QV_OK : QV_ERR_HIP;
}
