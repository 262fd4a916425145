// Greedy verification (Quasar, Sec. 4.5: the verifier's top-1 token decides; Sec. 4.2 /
// Table 1: the acceptance length counts the tokens a verify step emits).
//
// One launch: a grid of (chunks x M) workgroups scans the logits.  Each workgroup reduces its
// chunk of one row to a 64-bit key  (order(fp16 value) << 32) | (0xFFFFFFFF - index),  whose
// maximum is the largest value and, among equal values, the lowest index.  order() maps fp16
// bit patterns to integers monotonically and sends -0 and +0 to the same key, so they tie.
// Keys go to the workspace; the last workgroup of each row to arrive (one arrival counter per
// row, so no counter sees more than a row's chunks) reduces that row's keys and writes its
// argmax; the last row to finish (a second counter) then either scans a chain of drafts for the first mismatch (a
// wavefront ballot) or accepts a draft tree (Speculative Decoding Meets Quantization, review
// page: the target verifies a draft tree in one pass and keeps one path of it): a node is
// accepted when its parent is and its token equals the argmax at the parent, and the path
// runs from the root to the deepest accepted node, the lowest index among equals.
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 16384;  // logits per workgroup

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

// Tree inputs and outputs (TREE): per node its token and parent index (node 0 the root),
// the path of accepted node indices (-1 past its end), and {accept length, bonus token}.
struct TreeArgs {
  const int32_t* tokens;
  const int32_t* parent;
  int32_t* path;
  int32_t* accept;
};

template <bool TREE>
__global__ __launch_bounds__(kThreads) void verify_kernel(
    const uint16_t* __restrict__ logits, int M, int V, const int32_t* __restrict__ draft,
    int32_t* __restrict__ argmax_out, int32_t* __restrict__ n_accept_out,
    unsigned* __restrict__ counter, uint64_t* __restrict__ part, int32_t* __restrict__ rows,
    int chunks, TreeArgs tree) {
  const int c = blockIdx.x, m = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const uint16_t* row = logits + (size_t)m * V;
  const int beg = c * kChunk;
  const int end = min(beg + kChunk, V);
  // The tree's tokens and parents, loaded now so that the workgroup that ends up accepting
  // the tree does not wait on them (thread v < M holds node v).
  int my_tok = 0, my_par = 0;
  if constexpr (TREE) {
    if (tid < M) {
      my_tok = tree.tokens[tid];
      my_par = tree.parent[tid];
    }
  }

  uint64_t best = 0;
  if ((V & 7) == 0) {
    // All of the thread's 16-byte loads are issued before any is reduced (addresses past
    // the row's end are clamped to its start and their keys dropped).
    constexpr int kIters = kChunk / (kThreads * 8);
    u32x4 d[kIters];
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int e = beg + tid * 8 + i * kThreads * 8;
      d[i] = *reinterpret_cast<const u32x4*>(row + (e < end ? e : 0));
    }
#pragma unroll
    for (int i = 0; i < kIters; ++i) {
      const int e = beg + tid * 8 + i * kThreads * 8;
      if (e >= end) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint64_t k0 = make_key(d[i][j] & 0xFFFFu, e + 2 * j);
        const uint64_t k1 = make_key(d[i][j] >> 16, e + 2 * j + 1);
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
  // counter[1 + m]: chunks of row m; counter[0]: finished rows.
  if (!arrive_last(&counter[1 + m], (unsigned)chunks)) return;
  if (wave == 0) {
    uint64_t b = 0;
    for (int j = lane; j < chunks; j += kWave) {
      const uint64_t v = ld_coherent(&part[(size_t)m * chunks + j]);
      b = v > b ? v : b;
    }
    b = wave_max_u64(b);
    if (lane == 0) {
      const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
      argmax_out[m] = idx;
      st_coherent(&rows[m], idx);
    }
  }
  if (!arrive_last(&counter[0], (unsigned)M)) return;

  __shared__ int32_t amax[QV_MAX_M];
  if (tid < M) amax[tid] = ld_coherent(&rows[tid]);
  __syncthreads();
  if constexpr (!TREE) {
    if (wave == 0) {
      const bool miss = lane < M - 1 && draft[lane] != amax[lane];
      const uint64_t mask = __ballot(miss);
      if (lane == 0) {
        n_accept_out[0] = mask ? (int32_t)__builtin_ctzll(mask) : M - 1;
      }
    }
  } else {
    // At most 64 nodes, one lane of wave 0 each (node v in lane v).  A node is accepted when
    // its parent index is valid (0 <= parent < v), its token equals the argmax at its
    // parent, and its parent is accepted; the root always is.  Depth and acceptance along
    // the whole path come from pointer jumping over the parent links (six rounds of
    // shuffles, the root pointing to itself), which also leaves each lane its 2^j-th
    // ancestors; the path is the chain of ancestors of the deepest accepted node (the lowest
    // index among equals), and lane v is on it when its ancestor-of-best at its own depth
    // is v itself.
    __shared__ int32_t path[QV_MAX_M];
    __shared__ int32_t s_len;
    if (wave == 0) {
      const int v = lane;
      const bool valid = v < M && (v == 0 || (my_par >= 0 && my_par < v));
      int a = valid && v > 0 ? my_par : 0;
      bool acc = v == 0 || (valid && my_tok == amax[a]);
      int d = v == 0 ? 0 : 1;
      int up[6];
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        up[j] = a;
        const int da = __shfl(d, a, kWave);
        const int acca = __shfl((int)acc, a, kWave);
        const int aa = __shfl(a, a, kWave);
        d += da;
        acc = acc && acca != 0;
        a = aa;
      }
      const int key = acc ? (d << 6) | (63 - v) : -1;
      int kmax = key;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) kmax = max(kmax, __shfl_xor(kmax, off, kWave));
      const int best = 63 - (kmax & 63), len = kmax >> 6;
      // The ancestor of best that is len - d levels up (shuffles by every lane, selects after).
      const int steps = len - d;
      int t = best;
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int nt = __shfl(up[j], t, kWave);
        t = ((steps >> j) & 1) ? nt : t;
      }
      if (acc && steps >= 0 && t == v) path[d] = v;
      if (lane == 0) {
        s_len = len;
        tree.accept[0] = len;
        tree.accept[1] = amax[best];
      }
    }
    __syncthreads();
    if (tid < M) tree.path[tid] = tid <= s_len ? path[tid] : -1;
  }
}

}  // namespace

// Workspace after the counters: the chunk keys [M][chunks], then the rows' argmax [64].
size_t verify_partial_bytes(int M, int V) {
  const size_t chunks = ((size_t)V + kChunk - 1) / kChunk;
  return (size_t)M * chunks * sizeof(uint64_t) + QV_MAX_M * sizeof(int32_t);
}

hipError_t launch_verify(const uint16_t* logits, int M, int V, const int32_t* draft,
                         int32_t* argmax_out, int32_t* n_accept_out, unsigned* counters,
                         void* partials, hipStream_t stream) {
  const int chunks = (V + kChunk - 1) / kChunk;
  dim3 grid(chunks, M);
  uint64_t* keys = static_cast<uint64_t*>(partials);
  verify_kernel<false><<<grid, kThreads, 0, stream>>>(
      logits, M, V, draft, argmax_out, n_accept_out, counters, keys,
      reinterpret_cast<int32_t*>(keys + (size_t)M * chunks), chunks, TreeArgs{});
  return hipGetLastError();
}

hipError_t launch_verify_tree(const uint16_t* logits, int M, int V, const int32_t* tokens,
                              const int32_t* parent, int32_t* argmax_out, int32_t* path_out,
                              int32_t* accept_out, unsigned* counters, void* partials,
                              hipStream_t stream) {
  const int chunks = (V + kChunk - 1) / kChunk;
  dim3 grid(chunks, M);
  uint64_t* keys = static_cast<uint64_t*>(partials);
  verify_kernel<true><<<grid, kThreads, 0, stream>>>(
      logits, M, V, nullptr, argmax_out, nullptr, counters, keys,
      reinterpret_cast<int32_t*>(keys + (size_t)M * chunks), chunks,
      TreeArgs{tokens, parent, path_out, accept_out});
  return hipGetLastError();
}

}  // namespace qv
