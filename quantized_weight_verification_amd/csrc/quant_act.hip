// Per-token symmetric int8 activation quantisation (Quasar, Sec. 3.3 "Online Activation
// Smoothing and Quantization"): one workgroup per row; the row's absolute maximum is found
// with wavefront max-reductions (DPP/swizzle shuffles) and one LDS exchange between the
// four waves, then every element is divided by the row scale and rounded half-to-even.
//
// The row is read twice (once for the maximum, once to quantise); the second pass hits L2,
// since a row is at most 64 K elements.  Divisions are IEEE correctly rounded (the library
// is built with -fhip-fp32-correctly-rounded-divide-sqrt), so the codes are bit-identical
// to a plain scalar implementation of the same definition.
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

template <bool kSmooth>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ inv_smooth,
                                                             int K, int8_t* __restrict__ x_q,
                                                             float* __restrict__ x_scale) {
  const int m = blockIdx.x;
  const uint16_t* row = x + (size_t)m * K;
  int8_t* qrow = x_q + (size_t)m * K;
  const int nvec = K >> 3;

  float amax = 0.0f;
  for (int v = threadIdx.x; v < nvec; v += kThreads) {
    const f16x8 h = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(row + v * 8));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float f = (float)h[j];
      if (kSmooth) f = f * inv_smooth[v * 8 + j];
      amax = fmaxf(amax, fabsf(f));
    }
  }
  amax = wave_max(amax);
  __shared__ float red[kThreads / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const float s = amax / 127.0f;
  if (threadIdx.x == 0) x_scale[m] = s;

  for (int v = threadIdx.x; v < nvec; v += kThreads) {
    const f16x8 h = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(row + v * 8));
    uint32_t packed[2] = {0u, 0u};
    if (amax != 0.0f) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float f = (float)h[j];
        if (kSmooth) f = f * inv_smooth[v * 8 + j];
        float t = __builtin_rintf(f / s);
        t = fminf(fmaxf(t, -127.0f), 127.0f);
        packed[j >> 2] |= ((uint32_t)(int)t & 0xFFu) << (8 * (j & 3));
      }
    }
    *reinterpret_cast<u32x2*>(qrow + v * 8) = u32x2{packed[0], packed[1]};
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                            int8_t* x_q, float* x_scale, hipStream_t stream) {
  if (inv_smooth)
    quant_act_kernel<true><<<M, kThreads, 0, stream>>>(x, inv_smooth, K, x_q, x_scale);
  else
    quant_act_kernel<false><<<M, kThreads, 0, stream>>>(x, inv_smooth, K, x_q, x_scale);
  return hipGetLastError();
}

}  // namespace qv
