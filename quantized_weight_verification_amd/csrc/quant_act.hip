// Per-token symmetric int8 activation quantisation (Quasar, Sec. 3.3 "Online Activation
// Smoothing and Quantization"): each row is split into segments of one workgroup each; every
// workgroup finds the row's absolute maximum with wavefront max-reductions (DPP/swizzle
// shuffles) and one LDS exchange between its waves, then divides each element of its
// segment by the row scale and rounds half-to-even.
// The same kernel, reading bf16 rows, quantises weights offline per output channel (Quasar,
// Sec. 3.3 "Offline Weight Preparation": W_hat = Q(W diag(s)^-1), the column multipliers
// being the entries of diag(s)^-1), one row per workgroup of 128, 256 or 512 threads.
//
// Rows of up to 8 vectors per thread (32 K elements at 512 threads) are read once into
// registers (VPT 16-byte vectors per thread), so the kernel costs one HBM round trip plus the
// reduction; longer rows are read twice (the second pass hits L2).
// The element rules (quotient, rounding, clamping) live in quant_rules.h.
#include "qv_internal.h"
#include "quant_rules.h"

namespace qv {
namespace {

constexpr int kThreads = 512;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

template <int NTHR>
__device__ __forceinline__ float row_max(float amax) {
  amax = wave_max(amax);
  __shared__ float red[NTHR / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = amax;
  __syncthreads();
  float a = red[0];
#pragma unroll
  for (int i = 1; i < NTHR / kWave; ++i) a = fmaxf(a, red[i]);
  return a;
}

// NTHR threads per workgroup.  VPT > 0: the row lives in registers (nvec <= VPT * NTHR).
// VPT == 0: two passes.
// kSeg: long rows are split into gridDim.y segments: every workgroup of a row finds the
// absolute maximum of the whole row (the row is read from L2 by all but the first) and
// quantises only its segment, so the quantisation arithmetic of a row is spread over several
// CUs.  Without kSeg a workgroup quantises its whole row and the segment bounds (a division
// by gridDim.y among them) are compiled out: the one-row-per-workgroup weight preparation
// runs 12-14 % faster without them.
template <bool kSmooth, int VPT, bool kBf16, bool kSeg, int NTHR>
__global__ __launch_bounds__(NTHR) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ inv_smooth,
                                                             int K, int8_t* __restrict__ x_q,
                                                             float* __restrict__ x_scale) {
  const int m = blockIdx.x;
  const uint16_t* row = x + (size_t)m * K;
  int8_t* qrow = x_q + (size_t)m * K;
  const int nvec = K >> 3;
  const int segv = kSeg ? (nvec + gridDim.y - 1) / gridDim.y : nvec;  // vectors per segment
  const int v0 = kSeg ? blockIdx.y * segv : 0, v1 = kSeg ? min(v0 + segv, nvec) : nvec;

  float amax = 0.0f;
  u32x4 raw[VPT > 0 ? VPT : 1];
  if (VPT > 0) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = threadIdx.x + j * NTHR;
      raw[j] = v < nvec ? *reinterpret_cast<const u32x4*>(row + v * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = threadIdx.x + j * NTHR;
      if (v < nvec) amax = vec_absmax<kSmooth, kBf16>(raw[j], inv_smooth, v, amax);
    }
  } else {
    for (int v = threadIdx.x; v < nvec; v += NTHR)
      amax = vec_absmax<kSmooth, kBf16>(*reinterpret_cast<const u32x4*>(row + v * 8), inv_smooth, v, amax);
  }
  amax = row_max<NTHR>(amax);

  const float s = amax / 127.0f;
  const float rs = 1.0f / s;
  if (threadIdx.x == 0 && (!kSeg || blockIdx.y == 0)) x_scale[m] = s;

  if (VPT > 0) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = threadIdx.x + j * NTHR;
      if (v >= v0 && v < v1)
        *reinterpret_cast<u32x2*>(qrow + v * 8) = quantise8<kSmooth, kBf16>(raw[j], inv_smooth, v, amax, s, rs);
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += NTHR)
      *reinterpret_cast<u32x2*>(qrow + v * 8) = quantise8<kSmooth, kBf16>(
          *reinterpret_cast<const u32x4*>(row + v * 8), inv_smooth, v, amax, s, rs);
  }
}

// segs: workgroups per row (each quantises 1 / segs of it).
template <bool kSmooth, bool kBf16, bool kSeg, int NTHR = kThreads>
void launch_v(const uint16_t* x, const float* inv, int M, int K, int8_t* xq, float* xs,
              int segs, hipStream_t stream) {
  const int per = ((K >> 3) + NTHR - 1) / NTHR;  // vectors per thread
  const dim3 grid(M, segs);
  if (per <= 1)
    quant_act_kernel<kSmooth, 1, kBf16, kSeg, NTHR><<<grid, NTHR, 0, stream>>>(x, inv, K, xq, xs);
  else if (per <= 2)
    quant_act_kernel<kSmooth, 2, kBf16, kSeg, NTHR><<<grid, NTHR, 0, stream>>>(x, inv, K, xq, xs);
  else if (per <= 4)
    quant_act_kernel<kSmooth, 4, kBf16, kSeg, NTHR><<<grid, NTHR, 0, stream>>>(x, inv, K, xq, xs);
  else if (per <= 8)
    quant_act_kernel<kSmooth, 8, kBf16, kSeg, NTHR><<<grid, NTHR, 0, stream>>>(x, inv, K, xq, xs);
  else
    quant_act_kernel<kSmooth, 0, kBf16, kSeg, NTHR><<<grid, NTHR, 0, stream>>>(x, inv, K, xq, xs);
}

template <bool kSmooth, bool kBf16>
void launch_t(const uint16_t* x, const float* inv, int M, int K, int8_t* xq, float* xs,
              int segs, hipStream_t stream) {
  if (segs > 1)
    launch_v<kSmooth, kBf16, true>(x, inv, M, K, xq, xs, segs, stream);
  else
    launch_v<kSmooth, kBf16, false>(x, inv, M, K, xq, xs, 1, stream);
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                            int8_t* x_q, float* x_scale, hipStream_t stream, const Tuning& t) {
  // One workgroup per 1024 elements of a row: a few rows leave most CUs idle otherwise, and
  // the quantisation arithmetic after the row's maximum is on the launch's critical path
  // (measured inside a HIP graph at M = 8: K = 4096 2.70 -> 2.49 us with 4 workgroups per
  // row instead of 1, K = 12288 3.05 -> 2.83 us with 12 instead of 3, K = 28672 3.98 ->
  // about 3.7 us; a trivial kernel takes 1.6 us there).  Every workgroup of a row reads the
  // whole row, so with many rows the segments are capped at max(4, 128 / M): at M = 48,
  // K = 28672 (the Llama-3-70B down input) 9.3 -> 5.4 us with 4 instead of 28, K = 12288
  // 4.7 -> 3.7 us, K = 8192 3.7 -> 3.3 us; at M = 17, K = 28672, 5.9 -> 5.3 us with 4.
  int segs = (K + 1023) / 1024;
  const int cap = M > 32 ? 4 : 128 / M;
  if (segs > cap) segs = cap;
  if (int e = t(QV_TUNE_QUANT_SEGS)) segs = e;
  if (segs > (K >> 3)) segs = K >> 3;
  if (inv_smooth)
    launch_t<true, false>(x, inv_smooth, M, K, x_q, x_scale, segs, stream);
  else
    launch_t<false, false>(x, inv_smooth, M, K, x_q, x_scale, segs, stream);
  return hipGetLastError();
}

hipError_t launch_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K,
                             int8_t* w_q, float* w_scale, hipStream_t stream, const Tuning& t) {
  // One row per workgroup, the smallest workgroup that holds the row in registers at up to
  // 8 vectors per thread: smaller workgroups keep more rows in flight per CU (measured on
  // the Qwen3-8B shapes, K = 4096, against 512 threads: LM head 700-716 -> 557-608 us and
  // gate_up 103 -> 91 us with 128 threads, 610-660 / 92-93 us with 256).
  const int nvec = K >> 3;
  int thr = nvec <= 1024 ? 128 : nvec <= 2048 ? 256 : 512;
  if (int e = t(QV_TUNE_PREP_W8_THREADS)) thr = e <= 128 ? 128 : e <= 256 ? 256 : 512;
  if (thr == 128) {
    if (inv_s) launch_v<true, true, false, 128>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
    else launch_v<false, true, false, 128>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
  } else if (thr == 256) {
    if (inv_s) launch_v<true, true, false, 256>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
    else launch_v<false, true, false, 256>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
  } else {
    if (inv_s) launch_v<true, true, false, 512>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
    else launch_v<false, true, false, 512>(w_bf16, inv_s, N, K, w_q, w_scale, 1, stream);
  }
  return hipGetLastError();
}

}  // namespace qv
