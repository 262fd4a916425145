// Greedy verification (Quasar, Sec. 4.5: the verifier's top-1 token decides; Sec. 4.2 /
// Table 1: the acceptance length counts the tokens a verify step emits).
//
// One launch: a grid of (chunks x M) workgroups scans the logits.  Each workgroup reduces its
// chunk of one row to a 64-bit key  (order(fp16 value) << 32) | (0xFFFFFFFF - index),  whose
// maximum is the largest value and, among equal values, the lowest index.  order() maps fp16
// bit patterns to integers monotonically and sends -0 and +0 to the same key, so they tie.
// Keys go to the workspace; the last workgroup to arrive (arrival counter) reduces each row's
// keys, writes the argmax, and scans the drafts for the first mismatch (a wavefront ballot).
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;  // logits per workgroup

__device__ __forceinline__ uint32_t order16(uint32_t h) {
  if (h == 0x8000u) h = 0u;
  return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}

__device__ __forceinline__ uint64_t make_key(uint32_t h, uint32_t idx) {
  return ((uint64_t)order16(h) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void verify_kernel(
    const uint16_t* __restrict__ logits, int M, int V, const int32_t* __restrict__ draft,
    int32_t* __restrict__ argmax_out, int32_t* __restrict__ n_accept_out,
    unsigned* __restrict__ counter, uint64_t* __restrict__ part, int chunks) {
  const int c = blockIdx.x, m = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint16_t* row = logits + (size_t)m * V;
  const int beg = c * kChunk;
  const int end = min(beg + kChunk, V);

  uint64_t best = 0;
  if ((V & 7) == 0) {
    for (int e = beg + tid * 8; e < end; e += kThreads * 8) {
      const u32x4 d = *reinterpret_cast<const u32x4*>(row + e);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint64_t k0 = make_key(d[j] & 0xFFFFu, e + 2 * j);
        const uint64_t k1 = make_key(d[j] >> 16, e + 2 * j + 1);
        best = k0 > best ? k0 : best;
        best = k1 > best ? k1 : best;
      }
    }
  } else {
    for (int e = beg + tid; e < end; e += kThreads) {
      const uint64_t k = make_key(row[e], e);
      best = k > best ? k : best;
    }
  }
  best = wave_max_u64(best);
  __shared__ uint64_t red[kThreads / kWave];
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = red[0];
    for (int i = 1; i < kThreads / kWave; ++i) b = red[i] > b ? red[i] : b;
    st_coherent(&part[(size_t)m * chunks + c], b);
  }
  if (!arrive_last(counter, (unsigned)(M * chunks))) return;

  __shared__ int32_t amax[QV_MAX_M];
  for (int mm = wave; mm < M; mm += kThreads / kWave) {
    uint64_t b = 0;
    for (int j = lane; j < chunks; j += kWave) {
      const uint64_t v = ld_coherent(&part[(size_t)mm * chunks + j]);
      b = v > b ? v : b;
    }
    b = wave_max_u64(b);
    if (lane == 0) {
      const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
      amax[mm] = idx;
      argmax_out[mm] = idx;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const bool miss = lane < M - 1 && draft[lane] != amax[lane];
    const uint64_t mask = __ballot(miss);
    if (lane == 0) {
      n_accept_out[0] = mask ? (int32_t)__builtin_ctzll(mask) : M - 1;
    }
  }
}

}  // namespace

size_t verify_partial_bytes(int M, int V) {
  const size_t chunks = ((size_t)V + kChunk - 1) / kChunk;
  return (size_t)M * chunks * sizeof(uint64_t);
}

hipError_t launch_verify(const uint16_t* logits, int M, int V, const int32_t* draft,
                         int32_t* argmax_out, int32_t* n_accept_out, unsigned* counters,
                         void* partials, hipStream_t stream) {
  const int chunks = (V + kChunk - 1) / kChunk;
  dim3 grid(chunks, M);
  verify_kernel<<<grid, kThreads, 0, stream>>>(logits, M, V, draft, argmax_out, n_accept_out,
                                               counters, static_cast<uint64_t*>(partials), chunks);
  return hipGetLastError();
}

}  // namespace qv
