// W8A8 linear: int8 x int8 -> int32 on the gfx950 matrix cores, then dequantisation by the
// per-token and per-channel scales (Quasar, Sec. 3.3 "INT8 Gemm and Dequantization").
//
// Shape of the work: M (verified positions, <= 64) is tiny and N x K (the weights) is large,
// so the kernel is a weight stream bounded by HBM bandwidth.  Each workgroup owns one tile of
// 16 output channels and a K-slice; its waves split that slice further and stream their part
// of the 16 weight rows straight from HBM into VGPRs (one 16-byte load per lane per 64-wide
// K step, U steps in flight), feeding v_mfma_i32_16x16x64_i8 with
//   A = 16 weight rows x 64 k   (lane l: row l%16, bytes 16*(l/16) .. +16 of the K step)
//   B = 64 k x 16 tokens        (lane l: token l%16, the same 16 k)
// The activations are small and stay in L2.  Token columns past M read a valid row (row
// M-1) instead of branching; their outputs are never stored.  The waves' int32
// accumulators are summed through LDS (exact), and the epilogue applies
//   y = fp16( f32( f32(acc) * x_scale[m] ) * w_scale[n] )
// with round-to-nearest-even at each step.  With split-K (small N), each K-slice writes its
// int32 partial sums to the workspace and the last workgroup to arrive at the tile (arrival
// counter) adds them and runs the epilogue, then re-arms the counter.
#include "qv_internal.h"

namespace qv {
namespace {

__device__ __forceinline__ uint16_t dequant_epilogue(int32_t acc, float sx, float sw) {
  float t = (float)acc;
  t = t * sx;
  t = t * sw;
  return __builtin_bit_cast(uint16_t, (_Float16)t);
}

template <int MT, int U, int NW>
__global__ __launch_bounds__(NW * 64) void w8a8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int M, int K,
    const int8_t* __restrict__ w, const float* __restrict__ sw, int N,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, unsigned* __restrict__ counters,
    int32_t* __restrict__ part, int splits, int steps_per_split) {
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int kg = lane >> 4;
  const int n0 = tile * 16;

  const int steps_total = K >> 6;
  const int sb = split * steps_per_split;
  const int se = min(sb + steps_per_split, steps_total);
  const int ns = se - sb;
  const int s0 = sb + (ns * wave) / NW;
  const int s1 = sb + (ns * (wave + 1)) / NW;

  const int8_t* wp = w + (size_t)(n0 + r) * K + kg * 16;
  const int8_t* xp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xp[mt] = xq + (size_t)min(mt * 16 + r, M - 1) * K + kg * 16;

  i32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = i32x4{0, 0, 0, 0};

  int s = s0;
  for (; s + U <= s1; s += U) {
    i32x4 a[U];
    i32x4 b[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = *reinterpret_cast<const i32x4*>(wp + (size_t)(s + u) * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[mt][u] = *reinterpret_cast<const i32x4*>(xp[mt] + (size_t)(s + u) * 64);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[mt][u], acc[mt], 0, 0, 0);
  }
  for (; s < s1; ++s) {
    const i32x4 a = *reinterpret_cast<const i32x4*>(wp + (size_t)s * 64);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const i32x4 b = *reinterpret_cast<const i32x4*>(xp[mt] + (size_t)s * 64);
      acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[mt], 0, 0, 0);
    }
  }

  // Sum the waves' tiles through LDS.  The 16x16 accumulator tile puts output (i, j) with
  // i = 4*(l/16) + v (weight row), j = l%16 (token) in lane l, register v; store it as
  // red[wave][mt][j][i] so that consecutive threads of the reduction own consecutive n.
  __shared__ int32_t red[NW][MT][16][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<i32x4*>(&red[wave][mt][r][kg * 4]) = acc[mt];
  __syncthreads();

  for (int t = threadIdx.x; t < MT * 256; t += NW * 64) {
    const int mt = t >> 8, j = (t >> 4) & 15, i = t & 15;
    const int m = mt * 16 + j;
    if (m >= M) continue;
    int32_t sum = 0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) sum += red[wv][mt][j][i];
    const int n = n0 + i;
    if (splits == 1) {
      y[(size_t)m * N + n] = dequant_epilogue(sum, sx[m], sw[n]);
      if (acc_out) acc_out[(size_t)m * N + n] = sum;
    } else {
      part[((size_t)split * M + m) * N + n] = sum;
    }
  }
  if (splits == 1) return;

  // Split-K: the last workgroup of this tile adds the partial sums.
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) last = atomicAdd(&counters[tile], 1u) == (unsigned)(splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int t = threadIdx.x; t < MT * 256; t += NW * 64) {
    const int mt = t >> 8, j = (t >> 4) & 15, i = t & 15;
    const int m = mt * 16 + j;
    if (m >= M) continue;
    const int n = n0 + i;
    int32_t sum = 0;
    for (int sp = 0; sp < splits; ++sp) sum += part[((size_t)sp * M + m) * N + n];
    y[(size_t)m * N + n] = dequant_epilogue(sum, sx[m], sw[n]);
    if (acc_out) acc_out[(size_t)m * N + n] = sum;
  }
  if (threadIdx.x == 0) counters[tile] = 0u;
}

template <int MT, int U, int NW>
hipError_t launch_t(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                    const int8_t* w, const float* sw, int N, uint16_t* y, int32_t* acc_out,
                    unsigned* counters, void* partials, hipStream_t stream) {
  dim3 grid(p.tiles, p.splits);
  w8a8_kernel<MT, U, NW><<<grid, NW * 64, 0, stream>>>(
      xq, sx, M, K, w, sw, N, y, acc_out, counters, static_cast<int32_t*>(partials), p.splits,
      p.k_per_split / 64);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_w8a8(int M, int N, int K) {
  GemmPlan p{};
  p.waves = 4;
  if (int e = tune_env("QV_W8A8_WAVES")) p.waves = e == 8 ? 8 : 4;
  p.tiles = N / 16;
  const int steps = K / 64;
  // Aim for about four workgroups per CU (256 CUs) so every CU keeps weight loads in
  // flight; split K only when the output tiles alone cannot provide that.
  const int target = 1024;
  int splits = (target + p.tiles - 1) / p.tiles;
  const int max_splits = steps / p.waves > 0 ? steps / p.waves : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  if (int e = tune_env("QV_W8A8_SPLITS")) splits = e;
  if (splits > steps) splits = steps;
  if (p.tiles > QV_WORKSPACE_COUNTER_BYTES / 4) splits = 1;
  const int steps_per_split = (steps + splits - 1) / splits;
  splits = (steps + steps_per_split - 1) / steps_per_split;
  p.splits = splits;
  p.k_per_split = steps_per_split * 64;
  p.variant = (M + 15) / 16;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(int32_t) : 0;
  return p;
}

hipError_t launch_w8a8(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                       const int8_t* w, const float* sw, int N, uint16_t* y, int32_t* acc_out,
                       unsigned* counters, void* partials, hipStream_t stream) {
#define QV_W8A8_CASE(MT, U)                                                                   \
  case MT:                                                                                    \
    return p.waves == 8                                                                       \
               ? launch_t<MT, U, 8>(p, xq, sx, M, K, w, sw, N, y, acc_out, counters, partials, \
                                    stream)                                                   \
               : launch_t<MT, U, 4>(p, xq, sx, M, K, w, sw, N, y, acc_out, counters, partials, \
                                    stream);
  switch (p.variant) {
    QV_W8A8_CASE(1, 8)
    QV_W8A8_CASE(2, 4)
    QV_W8A8_CASE(3, 2)
    QV_W8A8_CASE(4, 2)
    default:
      return hipErrorInvalidValue;
  }
#undef QV_W8A8_CASE
}

}  // namespace qv
