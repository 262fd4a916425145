// Offline 4-bit weight preparation: bf16 weights [N][K] -> the group-128 asymmetric int4 format
// of the W4A16 / W4A8 linears (Speculative Decoding Meets Quantization, review page: 4-bit
// weight-quantised targets; the quantiser is this library's reading, the page giving none).
//
// Per group of 128 weights of one output channel:
//   lo = min(0, min w), hi = max(0, max w)       (the range always holds 0)
//   scale = fp16((hi - lo) / 15), or 1 if that rounds to 0
//   zero  = clamp(rint(-lo / scale), 0, 15)
//   code  = clamp(rint(w / scale) + zero, 0, 15)
// in fp32 with correctly rounded divisions and round-half-to-even; the codes are packed
// eight per 32-bit word, lowest k in the low nibble.
//
// Sixteen lanes own one group, eight consecutive weights (one 16-byte load, one output
// word) each; the group's range comes from four xor-shuffles inside the 16 lanes.  A
// 256-thread workgroup covers 64 groups, four per 16-lane set.  The pass reads 2 bytes and writes 0.52 bytes per
// weight, so it is bound by HBM bandwidth.
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerGroup = 16;

// Each 16-lane set takes kRep groups, kThreads / 16 sets per workgroup; all kRep loads of a
// lane are issued before the first group is quantised.
constexpr int kRep = 4;

__global__ __launch_bounds__(kThreads) void prepare_w4_kernel(const uint16_t* __restrict__ w,
                                                             int N, int K,
                                                             uint32_t* __restrict__ qweight,
                                                             uint16_t* __restrict__ scales,
                                                             uint8_t* __restrict__ zeros) {
  const int G = K / QV_W4A16_GROUP;
  const long total = (long)N * G;
  const int sets = kThreads / kLanesPerGroup;
  const long first = (long)blockIdx.x * sets * kRep + threadIdx.x / kLanesPerGroup;
  const int l = threadIdx.x % kLanesPerGroup;
  // Groups past the end repeat the last one (their lanes still take part in the shuffles)
  // and store nothing.
  u32x4 raw[kRep];
#pragma unroll
  for (int i = 0; i < kRep; ++i) {
    const long grp = first + (long)i * sets;
    const long gq = grp < total ? grp : total - 1;
    const long n = gq / G, g = gq - n * G;
    raw[i] = *reinterpret_cast<const u32x4*>(w + (size_t)n * K + (size_t)g * QV_W4A16_GROUP + l * 8);
  }
#pragma unroll
  for (int i = 0; i < kRep; ++i) {
    const long grp = first + (long)i * sets;
    const long gq = grp < total ? grp : total - 1;
    const long n = gq / G, g = gq - n * G;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t d = raw[i][j >> 1];
      x[j] = __builtin_bit_cast(float, (j & 1) ? (d & 0xFFFF0000u) : (d << 16));
    }
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo = fminf(lo, x[j]);
      hi = fmaxf(hi, x[j]);
    }
#pragma unroll
    for (int off = 1; off < kLanesPerGroup; off <<= 1) {
      lo = fminf(lo, __shfl_xor(lo, off, kWave));
      hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
    }
    _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
    if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
    const float s = (float)s16;
    const float z = fminf(fmaxf(__builtin_rintf(-lo / s), 0.0f), 15.0f);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float c = fminf(fmaxf(__builtin_rintf(x[j] / s) + z, 0.0f), 15.0f);
      word |= (uint32_t)c << (4 * j);
    }
    if (grp < total) {
      qweight[(size_t)n * (K / 8) + (size_t)g * (QV_W4A16_GROUP / 8) + l] = word;
      if (l == 0) {
        scales[(size_t)n * G + g] = __builtin_bit_cast(uint16_t, s16);
        zeros[(size_t)n * G + g] = (uint8_t)z;
      }
    }
  }
}

}  // namespace

hipError_t launch_prepare_w4(const uint16_t* w_bf16, int N, int K, uint32_t* qweight,
                             uint16_t* scales, uint8_t* zeros, hipStream_t stream) {
  const long groups = (long)N * (K / QV_W4A16_GROUP);
  const long per_block = (long)(kThreads / kLanesPerGroup) * kRep;
  const long blocks = (groups + per_block - 1) / per_block;
  prepare_w4_kernel<<<(unsigned)blocks, kThreads, 0, stream>>>(w_bf16, N, K, qweight, scales,
                                                               zeros);
  return hipGetLastError();
}

}  // namespace qv
