// W4A16 linear of the weight-only 4-bit verifier (Speculative Decoding Meets Quantization,
// review page, "The reading": a W4A16 target checks the draft in one forward pass).
//
// Weight format: code(n, k) = nibble k%8 of qweight[n][k/8] (low nibble first), group
// g = k/128 with an fp16 scale and a 0..15 zero point per (n, g); w = (code - zero) * scale.
//
// Dequantisation happens in registers, once per weight per pass, right before
// v_mfma_f32_16x16x32_f16:
//   * one 32-bit word holds 8 codes; (word >> 4i) & 0x000F000F | 0x64006400 turns codes i and
//     i+4 into the fp16 pair (1024 + code_i, 1024 + code_{i+4}) -- no conversion instruction;
//   * subtracting the pair (1024 + zero) is exact in fp16 (both lie in [1024, 1039]);
//   * one packed multiply by the scale rounds w to fp16 (the only rounding of the weight).
// The A operand of the MFMA (16 weight rows x 32 k) therefore takes its 8 k values per lane
// in the order 0,4,1,5,2,6,3,7 of the word; the activations are staged into LDS permuted the
// same way, so B (32 k x 16 tokens) lines up.  LDS rows are XOR-swizzled by 16-byte column so
// that the 16 token rows a wave reads at one column fall in distinct banks.
//
// Work split: a workgroup of NW waves owns NW*NT tiles of 16 output channels (each wave NT
// tiles) and one K-slice.  All its waves walk the slice together in chunks of 128*CG: the
// chunk's activations are staged into one of two LDS buffers while the previous chunk is
// computed, and the weights (plus scales and zeros) for the next chunk are loaded into
// registers before the current chunk's MFMAs, so HBM loads stay in flight across the single
// barrier per chunk.  All M <= 64 tokens live in the same wave (MT tiles of 16), so each
// weight is dequantised once no matter how many tokens are verified.  Split-K partial sums
// (fp32) go to the workspace and the last workgroup of a tile block adds them in split order,
// which keeps results bitwise reproducible.
#include "qv_internal.h"

namespace qv {
namespace {

// LDS-only barrier: waits for this wave's LDS traffic, not for its in-flight global loads.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// (a & mask) | bits in one VALU op.  gfx9 VOP3 encodings take no literal constants, so the
// compiler would otherwise split this into v_and_b32 + v_or_b32 with two literals.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(mask), "v"(bits));
  return d;
}

// Codes of one 32-bit word -> 8 fp16 weights (code - zero) * scale, in k order 0,4,1,5,2,6,3,7.
// zpair = (1024 + zero) twice, spair = scale twice, mask = 0x000F000F, magic = 0x64006400.
__device__ __forceinline__ f16x8 dequant8(uint32_t q, uint32_t zpair, uint32_t spair,
                                          uint32_t mask, uint32_t magic) {
  const f16x2 zz = __builtin_bit_cast(f16x2, zpair);
  const f16x2 ss = __builtin_bit_cast(f16x2, spair);
  const uint32_t v0 = and_or(q, mask, magic);
  const uint32_t v1 = and_or(q >> 4, mask, magic);
  const uint32_t v2 = and_or(q >> 8, mask, magic);
  const uint32_t v3 = and_or(q >> 12, mask, magic);
  const f16x2 h0 = (__builtin_bit_cast(f16x2, v0) - zz) * ss;
  const f16x2 h1 = (__builtin_bit_cast(f16x2, v1) - zz) * ss;
  const f16x2 h2 = (__builtin_bit_cast(f16x2, v2) - zz) * ss;
  const f16x2 h3 = (__builtin_bit_cast(f16x2, v3) - zz) * ss;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// (x0..x7) natural order -> (x0,x4,x1,x5,x2,x6,x3,x7), the order dequant8 produces.
__device__ __forceinline__ u32x4 permute_x(u32x4 d) {
  return u32x4{__builtin_amdgcn_perm(d.z, d.x, 0x05040100u), __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
               __builtin_amdgcn_perm(d.w, d.y, 0x05040100u), __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
}

template <int MT, int NT, int NW, int CG>
__global__ __launch_bounds__(NW * 64) void w4a16_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, unsigned* __restrict__ counters, float* __restrict__ part,
    int splits, int k_per_split) {
  constexpr int KC = 128 * CG;      // K per chunk
  constexpr int VPR = KC / 8;       // 16-byte vectors per staged row per chunk
  constexpr int NTHR = NW * 64;
  constexpr int ROWS = 16 * MT;     // staged token rows (>= M)
  constexpr int XV = (ROWS * VPR + NTHR - 1) / NTHR;  // staged vectors per thread
  __shared__ u32x4 xs[2][ROWS][VPR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3;  // 32-bit words per weight row
  const int G = K >> 7;   // groups per weight row
  const int kb = blockIdx.y * k_per_split;
  const int ke = min(kb + k_per_split, K);
  const int nchunks = (ke - kb + KC - 1) / KC;
  const uint32_t mask = 0x000F000Fu, magic = 0x64006400u;  // and_or takes them in VGPRs

  // This lane's weight rows: row 16*tile + r of each of the wave's NT tiles.
  const int tile0 = (blockIdx.x * NW + wave) * NT;
  bool tv[NT];
  const uint32_t* wrow[NT];
  const uint16_t* srow[NT];
  const uint8_t* zrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    tv[nt] = (tile0 + nt) * 16 < N;
    const int n = (tv[nt] ? (tile0 + nt) * 16 : 0) + r;
    wrow[nt] = qw + (size_t)n * KW + kg * 4;
    srow[nt] = scales + (size_t)n * G;
    zrow[nt] = zeros + (size_t)n * G;
  }

  u32x4 wcur[CG][NT], wnxt[CG][NT];
  uint32_t scur[CG][NT], snxt[CG][NT], zcur[CG][NT], znxt[CG][NT];
  u32x4 xr[XV];

  // Loads never branch: addresses past the slice (the last chunk) or past N (a partial tile
  // block) are clamped into the arrays, and what they bring is never used or stored.
  auto load_w = [&](int kc, u32x4 (&wr)[CG][NT], uint32_t (&sr)[CG][NT], uint32_t (&zr)[CG][NT]) {
#pragma unroll
    for (int gi = 0; gi < CG; ++gi) {
      const int g = min((kc >> 7) + gi, G - 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        wr[gi][nt] = *reinterpret_cast<const u32x4*>(wrow[nt] + (size_t)g * 16);
        sr[gi][nt] = srow[nt][g];
        zr[gi][nt] = zrow[nt][g];
      }
    }
  };
  // Token rows past M are staged from row M-1 and the columns past the slice from inside the
  // row; the products they feed land in outputs that are never stored or in skipped groups.
  auto load_x = [&](int kc) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = tid + j * NTHR;
      const int m = min(e / VPR, M - 1), v = e % VPR;
      const int k = min(kc + v * 8, K - 8);
      xr[j] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = tid + j * NTHR;
      const int m = e / VPR, v = e % VPR;
      if (e < ROWS * VPR) xs[buf][m][v ^ (m & 7)] = permute_x(xr[j]);
    }
  };

  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_w(kb, wcur, scur, zcur);
  load_x(kb);
  store_x(0);
  lds_barrier();

  for (int c = 0; c < nchunks; ++c) {
    const int kc = kb + c * KC;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_w(kc + KC, wnxt, snxt, znxt);
      load_x(kc + KC);
    }
    const int buf = c & 1;
#pragma unroll
    for (int gi = 0; gi < CG; ++gi) {
      if (kc + gi * 128 >= ke) break;
      uint32_t zp[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sp[nt] = scur[gi][nt] | (scur[gi][nt] << 16);
        const uint32_t zb = 0x6400u | zcur[gi][nt];
        zp[nt] = zb | (zb << 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 b[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          b[mt] = __builtin_bit_cast(f16x8, xs[buf][mt * 16 + r][(gi * 16 + kg * 4 + i) ^ (r & 7)]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f16x8 a = dequant8(wcur[gi][nt][i], zp[nt], sp[nt], mask, magic);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[mt], acc[nt][mt], 0, 0, 0);
        }
      }
    }
    if (more) store_x(buf ^ 1);
    lds_barrier();
    if (more) {
#pragma unroll
      for (int gi = 0; gi < CG; ++gi)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          wcur[gi][nt] = wnxt[gi][nt];
          scur[gi][nt] = snxt[gi][nt];
          zcur[gi][nt] = znxt[gi][nt];
        }
    }
  }

  // Output tile (16 channels x 16 tokens): lane l holds channels 4*(l/16)+v, token l%16.
  if (splits == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!tv[nt]) continue;
      const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        if (m >= M) continue;
        const f32x4 a = acc[nt][mt];
        const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[0], (_Float16)a[1]});
        const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[2], (_Float16)a[3]});
        *reinterpret_cast<u32x2*>(y + (size_t)m * N + n) = u32x2{lo, hi};
      }
    }
    return;
  }

#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
    const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m < M) *reinterpret_cast<f32x4*>(part + ((size_t)blockIdx.y * M + m) * N + n) = acc[nt][mt];
    }
  }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (tid == 0) last = atomicAdd(&counters[blockIdx.x], 1u) == (unsigned)(splits - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
    const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m >= M) continue;
      f32x4 s = *reinterpret_cast<const f32x4*>(part + (size_t)m * N + n);
      for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(part + ((size_t)sp * M + m) * N + n);
      const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)s[0], (_Float16)s[1]});
      const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)s[2], (_Float16)s[3]});
      *reinterpret_cast<u32x2*>(y + (size_t)m * N + n) = u32x2{lo, hi};
    }
  }
  if (tid == 0) counters[blockIdx.x] = 0u;
}

constexpr int kNW = 4;
constexpr int kNT = 2;
constexpr int kCG = 2;

template <int MT>
hipError_t launch_t(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                    const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                    unsigned* counters, void* partials, hipStream_t stream) {
  dim3 grid(p.tiles, p.splits);
  w4a16_kernel<MT, kNT, kNW, kCG><<<grid, kNW * 64, 0, stream>>>(
      x, M, K, qw, scales, zeros, N, y, counters, static_cast<float*>(partials), p.splits,
      p.k_per_split);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_w4a16(int M, int N, int K) {
  GemmPlan p{};
  p.waves = kNW;
  const int rows = kNW * kNT * 16;
  p.tiles = (N + rows - 1) / rows;  // tile blocks of `rows` channels
  const int groups = K / 128;
  const int target = 512;
  int splits = (target + p.tiles - 1) / p.tiles;
  const int max_splits = groups / (2 * kCG) > 0 ? groups / (2 * kCG) : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  if (int e = tune_env("QV_W4A16_SPLITS")) splits = e;
  if (splits > groups) splits = groups;
  if (p.tiles > QV_WORKSPACE_COUNTER_BYTES / 4) splits = 1;
  const int gps = (groups + splits - 1) / splits;
  splits = (groups + gps - 1) / gps;
  p.splits = splits;
  p.k_per_split = gps * 128;
  p.variant = (M + 15) / 16;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  return p;
}

hipError_t launch_w4a16(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream) {
  switch (p.variant) {
    case 1: return launch_t<1>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 2: return launch_t<2>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 3: return launch_t<3>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 4: return launch_t<4>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qv
