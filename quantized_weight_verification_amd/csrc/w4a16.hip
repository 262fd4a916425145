// W4A16 linear of the weight-only 4-bit verifier (Speculative Decoding Meets Quantization,
// review page, "The reading": a W4A16 target checks the draft in one forward pass).
//
// Weight format: code(n, k) = nibble k%8 of qweight[n][k/8] (low nibble first), group
// g = k/128 with an fp16 scale and a 0..15 zero point per (n, g); w = (code - zero) * scale.
//
// Dequantisation happens in registers, once per weight per pass, right before
// v_mfma_f32_16x16x32_f16:
//   * one 32-bit word holds 8 codes; masking a code into the mantissa of an fp16 with a fixed
//     exponent (1024 or 64) turns two codes at a time into exact fp16 values 1024 + c or
//     64 + c -- one shift and four and-or operations per word, no conversion instruction;
//   * subtracting the matching (1024 + zero) or (64 + zero) pair is exact in fp16;
//   * one packed multiply by the scale rounds w to fp16 (the only rounding of the weight).
// The A operand of the MFMA (16 weight rows x 32 k) therefore takes its 8 k values per lane
// in the order 0,4,1,5,2,6,3,7 of the word; the activations are staged into LDS permuted the
// same way, so B (32 k x 16 tokens) lines up.  The 16 vectors of each group of a staged row are
// permuted (swz) so that the 16 token rows x 4 lane quarters a wave reads at one K-step fall in
// distinct LDS banks.
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

// Masks and exponent bits of the code unpacking, held in registers.  (q & mask) | bits is one
// v_and_or_b32, but gfx9 VOP3 encodings take no literal constants, so with the constants
// visible the compiler splits it into v_and_b32 + v_or_b32; an empty asm at kernel start makes
// them opaque register values, and the compiler then selects v_and_or_b32 itself.  (Written
// as inline asm instead, the and-or's register writes were invisible to the compiler's hazard
// checks: when an MFMA whose unused result lanes it shared registers with was still in flight,
// the MFMA's late write-back clobbered the codes.)
struct UnpackK {
  uint32_t mlo, mhi, blo, bhi;
};
__device__ __forceinline__ UnpackK unpack_consts() {
  UnpackK k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
  asm volatile("" : "+v"(k.mlo), "+v"(k.mhi), "+v"(k.blo), "+v"(k.bhi));
  return k;
}
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  return (a & mask) | bits;
}

// Codes of one 32-bit word -> 8 fp16 weights (code - zero) * scale, in k order 0,4,1,5,2,6,3,7.
// A 16-bit half takes a code without shifting from two places: code bits 0-3 under the fp16
// exponent of 1024 (ulp 1) read as 1024 + code, and code bits 4-7 under the exponent of 64
// (ulp 1/16) read as 64 + code.  So one shift by 8 serves all four registers:
//   (q & 0x000F000F) | 0x6400 pair -> codes 0,4 as 1024 + c     (q >> 8): codes 2,6
//   (q & 0x00F000F0) | 0x5400 pair -> codes 1,5 as   64 + c     (q >> 8): codes 3,7
// Subtracting the matching (1024 + zero) or (64 + zero) pair is exact (both operands lie in
// one binade), and one packed multiply by the scale rounds w to fp16.
// zlo = (1024 + zero) twice, zhi = (64 + zero) twice, spair = scale twice.
__device__ __forceinline__ f16x8 dequant8(uint32_t q, uint32_t zlo, uint32_t zhi, uint32_t spair,
                                         const UnpackK& uk) {
  const uint32_t mlo = uk.mlo, mhi = uk.mhi, blo = uk.blo, bhi = uk.bhi;
  const f16x2 zl = __builtin_bit_cast(f16x2, zlo);
  const f16x2 zh = __builtin_bit_cast(f16x2, zhi);
  const f16x2 ss = __builtin_bit_cast(f16x2, spair);
  const uint32_t t = q >> 8;
  const uint32_t v0 = and_or(q, mlo, blo);
  const uint32_t v1 = and_or(q, mhi, bhi);
  const uint32_t v2 = and_or(t, mlo, blo);
  const uint32_t v3 = and_or(t, mhi, bhi);
  const f16x2 h0 = (__builtin_bit_cast(f16x2, v0) - zl) * ss;
  const f16x2 h1 = (__builtin_bit_cast(f16x2, v1) - zh) * ss;
  const f16x2 h2 = (__builtin_bit_cast(f16x2, v2) - zl) * ss;
  const f16x2 h3 = (__builtin_bit_cast(f16x2, v3) - zh) * ss;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Zero-point pairs for dequant8 from a zero in 0..15.
__device__ __forceinline__ uint32_t zero_lo(uint32_t z) {
  const uint32_t b = 0x6400u | z;
  return b | (b << 16);
}
__device__ __forceinline__ uint32_t zero_hi(uint32_t z) {
  const uint32_t b = 0x5400u | (z << 4);
  return b | (b << 16);
}

// Dequantisation operands of group p (0..7) of an 8-group block, from the block's scale vector
// sv (two fp16 scales per word) and zero vector zv (one zero point per byte): the scale twice,
// (1024 + z) twice and (64 + z) twice, one byte permute each.  Zero points are 0..15, so
// z << 4 stays inside its byte; the exponent bytes 0x64 and 0x54 are byte 1 of the unpacking
// constants.  (Built from shifts, masks and multiplies instead, these took about eight
// instructions per tile and group; at 48 tokens the chunk kernel is 1-3 % faster this way.)
__device__ __forceinline__ void group_pairs(const u32x4& sv, const u32x2& zv, int p,
                                            const UnpackK& uk, uint32_t& sp, uint32_t& zl,
                                            uint32_t& zh) {
  const uint32_t sw = sv[p >> 1], zw = zv[p >> 2];
  const uint32_t b = (uint32_t)(p & 3);
  sp = __builtin_amdgcn_perm(sw, sw, (p & 1) ? 0x03020302u : 0x01000100u);
  const uint32_t sel = 0x05000500u | (b << 16) | b;
  zl = __builtin_amdgcn_perm(uk.blo, zw, sel);
  zh = __builtin_amdgcn_perm(uk.bhi, zw << 4, sel);
}

// LDS position of logical 16-byte vector v of a staged token row m (v's group of 16 keeps its
// place; only the 16 positions inside it are permuted).  A fragment read by one wave takes, at
// one K-step i, vector 4 q + i (q the lane quarter) of 16 token rows: XORing the quarter with
// the row's two low bits and the step with its next two puts those 64 reads in distinct LDS
// banks on gfx950, where XORing the whole index with the row conflicts two ways (measured with
// ds_read_b128 at row strides of 512 B to 8 KB: 196-199 against 122-127 bytes per clock per CU).
__device__ __forceinline__ int swz(int m, int v) {
  return (v & ~15) | ((((m >> 2) ^ v) & 3) << 2) | ((m ^ (v >> 2)) & 3);
}

// (x0..x7) natural order -> (x0,x4,x1,x5,x2,x6,x3,x7), the order dequant8 produces.
__device__ __forceinline__ u32x4 permute_x(u32x4 d) {
  return u32x4{__builtin_amdgcn_perm(d.z, d.x, 0x05040100u), __builtin_amdgcn_perm(d.z, d.x, 0x07060302u),
               __builtin_amdgcn_perm(d.w, d.y, 0x05040100u), __builtin_amdgcn_perm(d.w, d.y, 0x07060302u)};
}

// Split-K finish for the workgroup that arrived last: y[m][n..n+3] for each of the lane's
// (tile, token tile) outputs is the sum over splits of the fp32 partials, added in split
// order (so results are reproducible).  The loads of four splits are issued together before
// any of them is added, so a split costs a fraction of a memory round trip, not one each.
// Rows past M and tiles past N read clamped in-bounds addresses and are not stored.
template <int NT, int MT>
__device__ __forceinline__ void finish_splits(const float* __restrict__ part, int splits, int M,
                                              int N, const int (&n)[NT], const bool (&tv)[NT],
                                              int r, uint16_t* __restrict__ y) {
  float t[NT][MT][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) t[nt][mt][q] = 0.f;
  for (int sp0 = 0; sp0 < splits; sp0 += 4) {
    float v[4][NT][MT][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sp = min(sp0 + j, splits - 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = min(mt * 16 + r, M - 1);
          const f32x4 a = ld_coherent_f4(&part[((size_t)sp * M + m) * N + n[nt]]);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[j][nt][mt][q] = a[q];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (sp0 + j >= splits) break;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) t[nt][mt][q] += v[j][nt][mt][q];
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m >= M) continue;
      const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)t[nt][mt][0], (_Float16)t[nt][mt][1]});
      const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)t[nt][mt][2], (_Float16)t[nt][mt][3]});
      *reinterpret_cast<u32x2*>(y + (size_t)m * N + n[nt]) = u32x2{lo, hi};
    }
  }
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

  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3;  // 32-bit words per weight row
  const int G = K >> 7;   // groups per weight row
  const int kb = blockIdx.y * k_per_split;
  const int ke = min(kb + k_per_split, K);
  const int nchunks = (ke - kb + KC - 1) / KC;

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
      uint32_t zl[NT], zh[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        sp[nt] = scur[gi][nt] | (scur[gi][nt] << 16);
        zl[nt] = zero_lo(zcur[gi][nt]);
        zh[nt] = zero_hi(zcur[gi][nt]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 b[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          b[mt] = __builtin_bit_cast(f16x8, xs[buf][mt * 16 + r][(gi * 16 + kg * 4 + i) ^ (r & 7)]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f16x8 a = dequant8(wcur[gi][nt][i], zl[nt], zh[nt], sp[nt], uk);
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

  float* mine = part + (size_t)blockIdx.y * M * N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
    const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m >= M) continue;
      st_coherent_f4(&mine[(size_t)m * N + n], acc[nt][mt]);
    }
  }
  if (!arrive_last(&counters[blockIdx.x], (unsigned)splits)) return;
  int nn[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) nn[nt] = (tv[nt] ? (tile0 + nt) * 16 : 0) + kg * 4;
  finish_splits<NT, MT>(part, splits, M, N, nn, tv, r, y);
}

// Ring variant.  The workgroup's K-slice of activations (all M rows) is staged into LDS
// once, permuted to the k order dequant8 produces, behind a single barrier; after that
// the main loop has no barrier and no global load other than the weight stream.  Each wave
// owns NT tiles of 16 channels and keeps the weight words, scales and zeros of the next P
// groups of 128 in flight in a register ring, refilling a slot as soon as its group has
// been consumed.  The activations come from LDS (lgkmcnt), so waiting for them never waits
// for the weight prefetches (vmcnt completes in order).  Split-K partial sums go through
// the workspace as in w4a16_kernel.
template <int MT, int NT, int NW, int P, bool VEC>
__global__ __launch_bounds__(NW * 64) void w4a16_ring_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, unsigned* __restrict__ counters, float* __restrict__ part,
    int splits, int groups_per_split) {
  static_assert(16 % P == 0, "P must divide the 16-group unroll");
  extern __shared__ u32x4 xs[];  // [M][VPR] 16-byte vectors, rows swizzled (swz)
  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3, G = K >> 7;
  const int gs0 = blockIdx.y * groups_per_split;
  const int gs1 = min(gs0 + groups_per_split, G);
  const int ng = gs1 - gs0;
  const int VPR = groups_per_split * 16;  // LDS row length in vectors (a multiple of 16)

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

  // Weight ring: slot p % P holds the words of group p (mod P).  Scales and zeros: with VEC
  // one 16-byte load brings the scales of 8 groups and one 8-byte load their zeros (slices
  // start at multiples of 8 groups, so blocks of 8 never straddle a slice); two block
  // buffers cover the P <= 8 groups in flight.  Without VEC they ride in the ring per group.
  u32x4 wq[P][NT];
  uint32_t sz[P][NT];
  u32x4 sblk[2][NT];
  u32x2 zblk[2][NT];
  auto load_w = [&](int g, int slot) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      wq[slot][nt] = *reinterpret_cast<const u32x4*>(wrow[nt] + (size_t)g * 16);
      if (!VEC) sz[slot][nt] = (uint32_t)srow[nt][g] | ((uint32_t)zrow[nt][g] << 16);
    }
  };
  auto load_blk = [&](int g, int b) {  // g: first group of an 8-block
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      sblk[b][nt] = *reinterpret_cast<const u32x4*>(srow[nt] + g);
      zblk[b][nt] = *reinterpret_cast<const u32x2*>(zrow[nt] + g);
    }
  };

  // Weight prologue first, so its latency overlaps the activation staging below.
  if (VEC) load_blk(gs0, 0);
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < ng) load_w(gs0 + p, p);

  // Staging: 8 loads in flight per thread per round (indices past the end re-read the
  // last vector and are not stored).
  const int nvec = M * ng * 16;
  for (int e0 = tid; e0 < nvec; e0 += 8 * NW * 64) {
    u32x4 d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = min(e0 + j * NW * 64, nvec - 1);
      const int m = e / (ng * 16), v = e - m * (ng * 16);
      d[j] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + (size_t)gs0 * 128 + v * 8);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = e0 + j * NW * 64;
      if (e < nvec) {
        const int m = e / (ng * 16), v = e - m * (ng * 16);
        xs[m * VPR + swz(m, v)] = permute_x(d[j]);
      }
    }
  }
  __syncthreads();

  // LDS vector index of this lane's B fragment for K-step i of group g is
  // boff[mt][i] + 16 g: the swizzle only permutes the 16 vectors of a group.
  int boff[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) boff[mt][i] = m * VPR + swz(m, kg * 4 + i);
  }

  f32x4 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int gl = 0; gl < ng; gl += 16) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int g = gl + p;  // group within the slice
      if (g < ng) {
        const int slot = p % P;
        uint32_t zl[NT], zh[NT], sp[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          uint32_t sb, zb;
          if (VEC) {
            const int b = (p >> 3) & 1, j = p & 7;
            sb = (sblk[b][nt][j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            zb = (zblk[b][nt][j >> 2] >> (8 * (j & 3))) & 0xFFu;
          } else {
            sb = sz[slot][nt] & 0xFFFFu;
            zb = sz[slot][nt] >> 16;
          }
          sp[nt] = sb | (sb << 16);
          zl[nt] = zero_lo(zb);
          zh[nt] = zero_hi(zb);
        }
        // The group entering the ring opens a new 8-block: fetch its scales and zeros.
        if (VEC && g + P < ng && ((p + P) & 7) == 0) load_blk(gs0 + g + P, ((p + P) >> 3) & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f16x8 bm[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) bm[mt] = __builtin_bit_cast(f16x8, xs[boff[mt][i] + g * 16]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const f16x8 a = dequant8(wq[slot][nt][i], zl[nt], zh[nt], sp[nt], uk);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bm[mt], acc[nt][mt], 0, 0, 0);
          }
        }
        // The slot's words are all unpacked: refill it with the group P ahead.
        if (g + P < ng) load_w(gs0 + g + P, slot);
      }
    }
  }

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

  float* mine = part + (size_t)blockIdx.y * M * N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
    const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m >= M) continue;
      st_coherent_f4(&mine[(size_t)m * N + n], acc[nt][mt]);
    }
  }
  if (!arrive_last(&counters[blockIdx.x], (unsigned)splits)) return;
  int nn[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) nn[nt] = (tv[nt] ? (tile0 + nt) * 16 : 0) + kg * 4;
  finish_splits<NT, MT>(part, splits, M, N, nn, tv, r, y);
}

// Chunked ring variant: the main W4A16 kernel whenever scales and zeros come as 8-group
// vectors.  Activations are staged in chunks of CG groups into two LDS buffers (so any M
// fits); the global loads of chunk c+2 are issued right after chunk c+1 has been written to
// LDS, a whole chunk ahead of their use.  One LDS-only barrier per chunk.  Weights come
// through a P-group register ring (a slot is refilled as soon as its group has been
// consumed); scales and zeros come as 8-group vectors, passed from a "next" to a "current"
// register block at every 8-group boundary.
//
// The host guarantees that every split holds a multiple of 8 groups, so the loop body (8
// groups) has no exits, and every global load in it is issued unconditionally (indices
// clamped to the last group or chunk; the surplus loads hit in cache and their data is
// never used).  The set and order of loads in flight is then the same on every path, so the
// compiler waits for exactly the load a step needs; a conditional load would make it drain
// all loads in flight at every iteration, which serialises memory latency and compute.
template <int MT, int NT, int NW, int P, int CG>
__global__ __launch_bounds__(NW * 64) void w4a16_chunk_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, unsigned* __restrict__ counters, float* __restrict__ part,
    int splits, int groups_per_split, int reduce_launch) {
  static_assert(8 % P == 0 && 8 % CG == 0, "P and CG divide the 8-group body");
  constexpr int VC = CG * 16;  // 16-byte vectors per token row per chunk
  constexpr int NTHR = NW * 64;
  constexpr int RB = 16 * MT * VC;  // vectors per LDS buffer: rows padded to whole token tiles
  constexpr int XV = (RB + NTHR - 1) / NTHR;  // staged vectors per thread
  constexpr bool EXACT = RB % NTHR == 0;      // every staging thread's vectors in range
  extern __shared__ u32x4 xs[];  // [2][16 MT][VC], rows swizzled (swz), + 1 spare vector
  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3, G = K >> 7;
  const int gs0 = blockIdx.y * groups_per_split;
  const int gs1 = min(gs0 + groups_per_split, G);
  const int ng = gs1 - gs0;  // a multiple of 8
  const int nch = ng / CG;

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
    srow[nt] = scales + (size_t)n * G + gs0;
    zrow[nt] = zeros + (size_t)n * G + gs0;
  }

  u32x4 wq[P][NT];
  u32x4 s_cur[NT], s_nxt[NT];
  u32x2 z_cur[NT], z_nxt[NT];
  auto load_w = [&](int g, int slot) {  // g relative to gs0
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wq[slot][nt] = *reinterpret_cast<const u32x4*>(wrow[nt] + (size_t)(gs0 + g) * 16);
  };
  auto load_blk = [&](int g) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_nxt[nt] = *reinterpret_cast<const u32x4*>(srow[nt] + g);
      z_nxt[nt] = *reinterpret_cast<const u32x2*>(zrow[nt] + g);
    }
  };
  // Chunk staging.  Thread tid owns vectors e = tid + j NTHR of the 16 MT x VC chunk layout
  // (row m = e / VC, vector v = e % VC); their global offsets (relative to the chunk start)
  // and swizzled LDS slots are fixed, so they are computed once.  Rows M .. 16 MT - 1 (the
  // padding of the last token tile) hold copies of row M - 1: finite values in token
  // columns whose outputs are never stored.  Vectors past the padded layout (when the
  // threads do not divide it) go to a spare LDS vector after the two buffers that nothing
  // reads: the stores stay unconditional, so the compiler cannot sink a load into a branch
  // next to its store (which would expose the load's whole latency).
  uint32_t goff[XV];
  int loff[XV];  // slot in buffer 0; in buffer 1 add RB (not for the spare vector)
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int e = tid + j * NTHR;
    const int m = e / VC, v = e % VC;  // VC is a power of two
    goff[j] = (uint32_t)min(m, M - 1) * (uint32_t)K + (uint32_t)v * 8u;
    loff[j] = e < RB ? m * VC + swz(m, v) : 2 * RB;
  }
  u32x4 xr[XV];
  auto load_chunk = [&](int c) {
    const uint16_t* base = x + (size_t)(gs0 + c * CG) * 128;
#pragma unroll
    for (int j = 0; j < XV; ++j) xr[j] = *reinterpret_cast<const u32x4*>(base + goff[j]);
  };
  auto store_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const bool in = EXACT || tid + j * NTHR < RB;
      xs[loff[j] + ((c & 1) && in ? RB : 0)] = permute_x(xr[j]);
    }
  };

  // The scheduling barriers keep the loads in this order (oldest first: scales and zeros,
  // then weights, then activations), the order the loop below expects them in.
  const int glast = ng - 1;
  load_blk(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_w(min(p, glast), p);
  __builtin_amdgcn_sched_barrier(0);
  load_chunk(0);
  store_chunk(0);
  load_chunk(min(1, nch - 1));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // LDS vector index of this lane's B fragment for token tile mt, K-step i of chunk-group gc
  // in buffer b: boff[i] + 16 VC mt + 16 gc + b RB.  The swizzle depends on a row's low four
  // bits only, so the token tiles differ by a constant offset (an immediate of the LDS read)
  // and the swizzle only permutes the 16 vectors of a group.
  int boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) boff[i] = r * VC + swz(r, kg * 4 + i);

  // Two accumulator sets per output tile, for even and odd K-steps, added at the end: the
  // MFMAs that feed one accumulator are then twice as far apart in the issue order (measured at
  // M = 48: gate_up 88.4 -> 85.5 us, down 49.6 -> 48.2).  Only while the registers allow it
  // (at eight tiles per wave the second set would spill).
  constexpr bool ACC2 = NT * MT <= 6;
  f32x4 acc[NT][MT], acc2[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc2[nt][mt] = acc[nt][mt];
    }

  f16x8 bn[MT];  // the B fragments of the next K-step
  auto read_b = [&](const u32x4* buf, int i, f16x8 (&b)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) b[mt] = __builtin_bit_cast(f16x8, buf[boff[i] + 16 * VC * mt]);
  };

  // One 8-group body.  The first body is peeled off the loop: the compiler may reorder the
  // prologue's loads, and only the loop's own order should decide the loop's waits.
  auto body = [&](int gb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_cur[nt] = s_nxt[nt];
      z_cur[nt] = z_nxt[nt];
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int g = gb + p;
      const int slot = p % P;
      uint32_t zl[NT], zh[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) group_pairs(s_cur[nt], z_cur[nt], p, uk, sp[nt], zl[nt], zh[nt]);
      if (p == 8 - P) {  // the next body's scales and zeros
        load_blk(min(gb + 8, ng - 8));
        __builtin_amdgcn_sched_barrier(0);
      }
      const u32x4* buf = xs + ((g / CG) & 1) * RB + (p % CG) * 16;
      // B fragments are read one K-step ahead of their MFMAs (within a chunk: the next
      // chunk is readable only after the barrier at the end of this one); left to itself the
      // compiler reads each step's fragments right before its MFMAs and waits for them there.
      if (p % CG == 0) read_b(buf, 0, bn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 bm[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) bm[mt] = bn[mt];
        if (i < 3) read_b(buf, i + 1, bn);
        else if (p % CG != CG - 1) read_b(buf + 16, 0, bn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // The dequantisation runs at raised wave priority, so that a wave with weights in
          // hand wins the VALU over one that is issuing MFMAs, whose matrix-core work then
          // overlaps it (measured at M = 48: qkv 23.0 -> 22.4 us, gate_up 83.1 -> 81.3,
          // down 48.1 -> 46.7; raising it around the MFMAs instead changed nothing).
          __builtin_amdgcn_s_setprio(1);
          const f16x8 a = dequant8(wq[slot][nt][i], zl[nt], zh[nt], sp[nt], uk);
          __builtin_amdgcn_s_setprio(0);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (ACC2 && (i & 1)) acc2[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bm[mt], acc2[nt][mt], 0, 0, 0);
            else acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bm[mt], acc[nt][mt], 0, 0, 0);
        }
      }
      load_w(min(g + P, glast), slot);  // the slot's words are all unpacked
      // Keep the refill here: the scheduler would otherwise bunch the refills of several
      // groups together late in the body, leaving the ring nearly empty in between.
      __builtin_amdgcn_sched_barrier(0);
      if (p % CG == CG - 1) {           // end of chunk g / CG
        const int c = g / CG;
        // Chunk c+1 into the buffer chunk c-1 used (every wave is past that chunk's barrier);
        // after the last chunk this writes data nobody reads.
        store_chunk(c + 1);
        load_chunk(min(c + 2, nch - 1));
        lds_barrier();
      }
    }
  };
  body(0);
  for (int gb = 8; gb < ng; gb += 8) body(gb);
  if (ACC2) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] += acc2[nt][mt];
  }

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

  float* mine = part + (size_t)blockIdx.y * M * N;
  if (reduce_launch) {  // a second launch adds the splits: plain stores, nothing to wait for
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (!tv[nt]) continue;
      const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + r;
        if (m >= M) continue;
        *reinterpret_cast<f32x4*>(&mine[(size_t)m * N + n]) = acc[nt][mt];
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
      if (m >= M) continue;
      st_coherent_f4(&mine[(size_t)m * N + n], acc[nt][mt]);
    }
  }
  if (!arrive_last(&counters[blockIdx.x], (unsigned)splits)) return;
  int nn[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) nn[nt] = (tv[nt] ? (tile0 + nt) * 16 : 0) + kg * 4;
  finish_splits<NT, MT>(part, splits, M, N, nn, tv, r, y);
}

// Chunked variant with a staging wave: NW compute waves as in w4a16_chunk_kernel plus one
// wave (the last) that only moves the activation chunks from global memory into the two LDS
// buffers, so the compute waves issue no staging loads, permutes or LDS stores.  With 7
// compute waves the staging wave takes the eighth slot of a CU at two waves per SIMD, which
// the 7-wave chunk kernel left empty.  (Measured at 48 tokens on the Llama-3-70B gate_up: the
// chunk kernel's compute alone, weights from registers, takes 57 us without its staging and
// 69 us with it; this kernel takes 4-6 % less time than the chunk kernel in full.  A deeper
// weight ring in the registers the staging freed was slower, P = 8 against 4.)
// Every wave passes the same barriers: one after the prologue, one at the end of each chunk.
// The staging wave stores chunk c + 1 (loaded during chunk c - 1) right after the barrier
// that ends chunk c - 1, when no wave reads that buffer any more, then loads chunk c + 2.
// The compute waves issue the next body's scales and zeros a whole body ahead and leave the
// wave priority alone (both measured 1-2 % faster here, where the chunk kernel gains from
// raising it).  The split-K partials, if any, always go to a second launch (the in-kernel
// finish would need the staging wave at its barriers).
template <int MT, int NT, int NW, int P, int CG>
__global__ __launch_bounds__((NW + 1) * 64) void w4a16_stage_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, float* __restrict__ part, int splits, int groups_per_split) {
  static_assert(8 % P == 0 && 8 % CG == 0, "P and CG divide the 8-group body");
  constexpr int VC = CG * 16;       // 16-byte vectors per token row per chunk
  constexpr int RB = 16 * MT * VC;  // vectors per LDS buffer: rows padded to whole token tiles
  constexpr int XV = RB / 64;       // vectors per staging lane
  static_assert(RB % 64 == 0 && XV <= 48, "one staging wave holds a whole chunk");
  extern __shared__ u32x4 xs[];  // [2][16 MT][VC], rows swizzled (swz)
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int KW = K >> 3, G = K >> 7;
  const int gs0 = blockIdx.y * groups_per_split;
  const int gs1 = min(gs0 + groups_per_split, G);
  const int ng = gs1 - gs0;  // a multiple of 8
  const int nch = ng / CG;

  if (wave == NW) {
    // Vector e = lane + 64 j of the 16 MT x VC chunk layout: row m = e / VC, vector v = e % VC
    // (rows M .. 16 MT - 1 copy row M - 1, finite values in columns nobody stores).  Step j
    // covers RPJ rows from row m0 (the same for the whole wave), so a load takes the row's
    // address as a wave-uniform base plus a 32-bit lane offset.
    constexpr int RPJ = VC >= 64 ? 1 : 64 / VC;
    const int sub = RPJ == 1 ? 0 : lane / VC;
    const int vl = RPJ == 1 ? lane : lane % VC;
    u32x4 xr[XV];
    auto load_chunk = [&](int c) {
      const uint16_t* base = x + (size_t)(gs0 + c * CG) * 128;
#pragma unroll
      for (int j = 0; j < XV; ++j) {
        const int m0 = RPJ == 1 ? 64 * j / VC : RPJ * j;
        const int v = RPJ == 1 ? 64 * j % VC + vl : vl;
        const uint16_t* row0 = base + (size_t)min(m0, M - 1) * K;
        const int d = RPJ == 1 ? 0 : (min(m0 + sub, M - 1) - min(m0, M - 1)) * K;
        xr[j] = *reinterpret_cast<const u32x4*>(row0 + d + v * 8);
      }
    };
    auto store_chunk = [&](int c) {
      u32x4* buf = xs + (c & 1) * RB;
#pragma unroll
      for (int j = 0; j < XV; ++j) {
        const int m = (RPJ == 1 ? 64 * j / VC : RPJ * j) + sub;
        const int v = RPJ == 1 ? 64 * j % VC + vl : vl;
        buf[m * VC + swz(m, v)] = permute_x(xr[j]);
      }
    };
    load_chunk(0);
    store_chunk(0);
    load_chunk(min(1, nch - 1));
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      // Chunk c + 1 into the buffer chunk c - 1 used; after the last chunk this writes data
      // nobody reads.
      store_chunk(c + 1);
      load_chunk(min(c + 2, nch - 1));
      lds_barrier();
    }
    return;
  }

  const UnpackK uk = unpack_consts();
  const int r = lane & 15, kg = lane >> 4;
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
    srow[nt] = scales + (size_t)n * G + gs0;
    zrow[nt] = zeros + (size_t)n * G + gs0;
  }

  u32x4 wq[P][NT];
  u32x4 s_cur[NT], s_nxt[NT];
  u32x2 z_cur[NT], z_nxt[NT];
  auto load_w = [&](int g, int slot) {  // g relative to gs0
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wq[slot][nt] = *reinterpret_cast<const u32x4*>(wrow[nt] + (size_t)(gs0 + g) * 16);
  };
  auto load_blk = [&](int g) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_nxt[nt] = *reinterpret_cast<const u32x4*>(srow[nt] + g);
      z_nxt[nt] = *reinterpret_cast<const u32x2*>(zrow[nt] + g);
    }
  };
  const int glast = ng - 1;
  load_blk(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_w(min(p, glast), p);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // B fragment of token tile mt, K-step i of chunk-group gc in buffer b: boff[i] + 16 VC mt +
  // 16 gc + b RB (as in w4a16_chunk_kernel).
  int boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) boff[i] = r * VC + swz(r, kg * 4 + i);

  constexpr bool ACC2 = NT * MT <= 6;
  f32x4 acc[NT][MT], acc2[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc2[nt][mt] = acc[nt][mt];
    }

  f16x8 bn[MT];
  auto read_b = [&](const u32x4* buf, int i, f16x8 (&b)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) b[mt] = __builtin_bit_cast(f16x8, buf[boff[i] + 16 * VC * mt]);
  };

  auto body = [&](int gb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_cur[nt] = s_nxt[nt];
      z_cur[nt] = z_nxt[nt];
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int g = gb + p;
      const int slot = p % P;
      uint32_t zl[NT], zh[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) group_pairs(s_cur[nt], z_cur[nt], p, uk, sp[nt], zl[nt], zh[nt]);
      if (p == 0) {  // the next body's scales and zeros, a whole body ahead
        load_blk(min(gb + 8, ng - 8));
        __builtin_amdgcn_sched_barrier(0);
      }
      const u32x4* buf = xs + ((g / CG) & 1) * RB + (p % CG) * 16;
      if (p % CG == 0) read_b(buf, 0, bn);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f16x8 bm[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) bm[mt] = bn[mt];
        if (i < 3) read_b(buf, i + 1, bn);
        else if (p % CG != CG - 1) read_b(buf + 16, 0, bn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f16x8 a = dequant8(wq[slot][nt][i], zl[nt], zh[nt], sp[nt], uk);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (ACC2 && (i & 1)) acc2[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bm[mt], acc2[nt][mt], 0, 0, 0);
            else acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bm[mt], acc[nt][mt], 0, 0, 0);
        }
      }
      load_w(min(g + P, glast), slot);
      __builtin_amdgcn_sched_barrier(0);
      if (p % CG == CG - 1) lds_barrier();  // end of chunk g / CG
    }
  };
  body(0);
  for (int gb = 8; gb < ng; gb += 8) body(gb);
  if (ACC2) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[nt][mt] += acc2[nt][mt];
  }

  float* mine = part + (size_t)blockIdx.y * M * N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tv[nt]) continue;
    const int n = (tile0 + nt) * 16 + kg * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + r;
      if (m >= M) continue;
      const f32x4 a = acc[nt][mt];
      if (splits == 1) {
        const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[0], (_Float16)a[1]});
        const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[2], (_Float16)a[3]});
        *reinterpret_cast<u32x2*>(y + (size_t)m * N + n) = u32x2{lo, hi};
      } else {
        *reinterpret_cast<f32x4*>(&mine[(size_t)m * N + n]) = a;
      }
    }
  }
}

// Wide variant (reached by configuration override; the kernel with a staging wave is 6 % faster
// at 17 to 32 tokens on gate_up-sized linears, where this one was the plan before it): the same
// chunked activation staging, weight ring and 8-group scale/zero vectors as w4a16_chunk_kernel, on
// v_mfma_f32_32x32x16_f16 with tiles of 32 channels and 32 tokens.  Chip-wide probes on gfx950
// put that instruction at 1.94 PFLOP/s against 1.22-1.33 for the 16x16x32 one, and 32 packed-
// fp16 VALU instructions next to every 4 of them cost 9 % more time where next to 8 of the
// 16x16x32 ones they cost 44 %.  In the kernel that buys less than the probes suggest: at 17-32
// tokens the Llama-3-70B gate_up is 0.5-9 % faster than on the chunk kernel (two boxes: 70.5-72.1
// against 75.8-77.4 us, 73.4-75.9 against 73.8-77.6), the three narrower linears are not, and at
// 48 tokens (64 padded) every shape tried was slower (92.6-136 against 83.1 us for gate_up).
//
template <int MT, int NT, int NW, int P, int CG>
__global__ __launch_bounds__(NW * 64) void w4a16_wide_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, float* __restrict__ part, int splits, int groups_per_split) {
  static_assert(8 % P == 0 && 8 % CG == 0, "P and CG divide the 8-group body");
  constexpr int VC = CG * 16;                 // 16-byte vectors per token row per chunk
  constexpr int NTHR = NW * 64;
  constexpr int RB = 32 * MT * VC;            // vectors per LDS buffer (rows padded to 32 MT)
  constexpr int XV = (RB + NTHR - 1) / NTHR;  // staged vectors per thread
  constexpr bool EXACT = RB % NTHR == 0;
  extern __shared__ u32x4 xs[];  // [2][32 MT][VC], rows swizzled, + 1 spare vector
  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, c = lane & 31, h = lane >> 5;
  const int KW = K >> 3, G = K >> 7;
  const int gs0 = blockIdx.y * groups_per_split;
  const int gs1 = min(gs0 + groups_per_split, G);
  const int ng = gs1 - gs0;  // a multiple of 8
  const int nch = ng / CG;

  const int tile0 = (blockIdx.x * NW + wave) * NT;  // 32-channel tiles
  int n0[NT];
  const uint32_t* wrow[NT];
  const uint16_t* srow[NT];
  const uint8_t* zrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    n0[nt] = (tile0 + nt) * 32;
    const int n = n0[nt] + c < N ? n0[nt] + c : N - 1;
    wrow[nt] = qw + (size_t)n * KW + h * 8;
    srow[nt] = scales + (size_t)n * G + gs0;
    zrow[nt] = zeros + (size_t)n * G + gs0;
  }

  u32x4 wq[P][NT][2];
  u32x4 s_cur[NT], s_nxt[NT];
  u32x2 z_cur[NT], z_nxt[NT];
  auto load_w = [&](int g, int slot) {  // g relative to gs0
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t* src = wrow[nt] + (size_t)(gs0 + g) * 16;
      wq[slot][nt][0] = *reinterpret_cast<const u32x4*>(src);
      wq[slot][nt][1] = *reinterpret_cast<const u32x4*>(src + 4);
    }
  };
  auto load_blk = [&](int g) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_nxt[nt] = *reinterpret_cast<const u32x4*>(srow[nt] + g);
      z_nxt[nt] = *reinterpret_cast<const u32x2*>(zrow[nt] + g);
    }
  };
  // Chunk staging as in w4a16_chunk_kernel: fixed per-thread global offsets and LDS slots;
  // rows M .. 32 MT - 1 copy row M - 1; vectors past the padded layout go to a spare slot.
  uint32_t goff[XV];
  int loff[XV];
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int e = tid + j * NTHR;
    const int m = e / VC, v = e % VC;
    goff[j] = (uint32_t)min(m, M - 1) * (uint32_t)K + (uint32_t)v * 8u;
    loff[j] = e < RB ? m * VC + (v ^ (m & 15)) : 2 * RB;
  }
  u32x4 xr[XV];
  auto load_chunk = [&](int ch) {
    const uint16_t* base = x + (size_t)(gs0 + ch * CG) * 128;
#pragma unroll
    for (int j = 0; j < XV; ++j) xr[j] = *reinterpret_cast<const u32x4*>(base + goff[j]);
  };
  auto store_chunk = [&](int ch) {
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const bool in = EXACT || tid + j * NTHR < RB;
      xs[loff[j] + ((ch & 1) && in ? RB : 0)] = permute_x(xr[j]);
    }
  };

  const int glast = ng - 1;
  load_blk(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_w(min(p, glast), p);
  __builtin_amdgcn_sched_barrier(0);
  load_chunk(0);
  store_chunk(0);
  load_chunk(min(1, nch - 1));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // LDS vector index of this lane's B fragment for token tile mt, K-step j of chunk-group gc
  // in buffer b: boff[j] + 32 VC mt + 16 gc + b RB (row c + 32 mt has the swizzle of row c).
  int boff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) boff[j] = c * VC + ((8 * h + j) ^ (c & 15));

  f32x16 acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][mt][r] = 0.f;

  f16x8 bn[MT];  // the B fragments of the next K-step
  auto read_b = [&](const u32x4* buf, int j, f16x8 (&b)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) b[mt] = __builtin_bit_cast(f16x8, buf[boff[j] + 32 * VC * mt]);
  };

  auto body = [&](int gb) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_cur[nt] = s_nxt[nt];
      z_cur[nt] = z_nxt[nt];
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int g = gb + p;
      const int slot = p % P;
      uint32_t zl[NT], zh[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) group_pairs(s_cur[nt], z_cur[nt], p, uk, sp[nt], zl[nt], zh[nt]);
      if (p == 8 - P) {  // the next body's scales and zeros
        load_blk(min(gb + 8, ng - 8));
        __builtin_amdgcn_sched_barrier(0);
      }
      const u32x4* buf = xs + ((g / CG) & 1) * RB + (p % CG) * 16;
      if (p % CG == 0) read_b(buf, 0, bn);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        f16x8 bm[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) bm[mt] = bn[mt];
        if (j < 7) read_b(buf, j + 1, bn);
        else if (p % CG != CG - 1) read_b(buf + 16, 0, bn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const f16x8 a = dequant8(wq[slot][nt][j >> 2][j & 3], zl[nt], zh[nt], sp[nt], uk);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bm[mt], acc[nt][mt], 0, 0, 0);
        }
      }
      load_w(min(g + P, glast), slot);  // the slot's words are all unpacked
      __builtin_amdgcn_sched_barrier(0);
      if (p % CG == CG - 1) {  // end of chunk g / CG
        const int ch = g / CG;
        store_chunk(ch + 1);
        load_chunk(min(ch + 2, nch - 1));
        lds_barrier();
      }
    }
  };
  body(0);
  for (int gb = 8; gb < ng; gb += 8) body(gb);

  // Register r of this lane: channel n0 + 8 (r / 4) + 4 h + r % 4, token c + 32 mt; four
  // consecutive channels per quarter rb = r / 4, stored together.
  float* mine = part + (size_t)blockIdx.y * M * N;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 32 + c;
      if (m >= M) continue;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int n = n0[nt] + 8 * rb + 4 * h;
        if (n >= N) continue;
        const f32x16& a = acc[nt][mt];
        if (splits == 1) {
          const uint32_t lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[4 * rb], (_Float16)a[4 * rb + 1]});
          const uint32_t hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)a[4 * rb + 2], (_Float16)a[4 * rb + 3]});
          *reinterpret_cast<u32x2*>(y + (size_t)m * N + n) = u32x2{lo, hi};
        } else {
          *reinterpret_cast<f32x4*>(&mine[(size_t)m * N + n]) =
              f32x4{a[4 * rb], a[4 * rb + 1], a[4 * rb + 2], a[4 * rb + 3]};
        }
      }
    }
  }
}

// Codes of one 32-bit word -> fp16 pairs without zero point or scale, in the order of
// dequant8: codes 0,4 and 2,6 as 1024 + c, codes 1,5 and 3,7 as 64 + c (exact), as the four
// 32-bit halves of the MFMA operand.  The result is assembled from scalars: reading the
// components of a vector built from the and-or results back out (u.y, u.z, u.w) was
// miscompiled to u.x by this compiler when the components then fed fp16 pair arithmetic.
__device__ __forceinline__ u32x4 unpack8(uint32_t q, const UnpackK& uk) {
  const uint32_t t = q >> 8;
  const uint32_t u0 = and_or(q, uk.mlo, uk.blo);
  const uint32_t u1 = and_or(q, uk.mhi, uk.bhi);
  const uint32_t u2 = and_or(t, uk.mlo, uk.blo);
  const uint32_t u3 = and_or(t, uk.mhi, uk.bhi);
  return u32x4{u0, u1, u2, u3};
}

// Codes of one word -> the exact fp16 differences code - zero, from the (1024 + z, 64 + z)
// pairs zl and zh: one packed subtraction per pair, each within one binade (exact).
__device__ __forceinline__ u32x4 unpack8_minus_zero(uint32_t q, uint32_t zl, uint32_t zh,
                                                   const UnpackK& uk) {
  const uint32_t t = q >> 8;
  const f16x2 lo = __builtin_bit_cast(f16x2, zl), hi = __builtin_bit_cast(f16x2, zh);
  const uint32_t d0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(q, uk.mlo, uk.blo)) - lo);
  const uint32_t d1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(q, uk.mhi, uk.bhi)) - hi);
  const uint32_t d2 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(t, uk.mlo, uk.blo)) - lo);
  const uint32_t d3 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, and_or(t, uk.mhi, uk.bhi)) - hi);
  return u32x4{d0, d1, d2, d3};
}

// Zero point z of group p (0..7) of an 8-group zero vector, as z | z << 16: one byte permute.
__device__ __forceinline__ uint32_t zero_pair(u32x2 zv, int p) {
  const uint32_t b = (uint32_t)(p & 3);
  return __builtin_amdgcn_perm(0u, zv[p >> 2], 0x0C000C00u | (b << 16) | b);
}

// W4A16 for one token tile (M <= 16): sequential verification of a draft.
//
// The MFMA takes the activations as its A operand (16 token rows x 32 k) and the unpacked
// codes as its B operand (32 k x 16 channels), so lane l accumulates D[token 4(l/16)+v]
// [channel l%16] -- the channel whose codes, scale and zero point the lane itself loads.  The
// MFMAs of each 128-group start from zero and the group's sum enters the fp32 result through
// one FMA with the group's scale:
//   y[m][n] = sum_g s[n][g] * sum_{k in g} x[m][k] * (code(n, k) - z[n][g])
// The codes enter as the exact fp16 values 1024 + c or 64 + c (one and-or per two codes, no
// conversion).  The offset and the zero point leave either by an exact fp16 subtraction of
// the (1024 + z, 64 + z) pairs before the MFMA (FOLD = false), or by a second MFMA per K-step
// against the constant pairs -(1024 + z), -(64 + z) (FOLD = true), which trades the four
// subtractions per word for matrix-core work that is idle at this M.  No weight is rounded:
// c - z is exact and the scale multiplies the group sum in fp32.  Per word of 8 codes this
// leaves 5 (FOLD) or 9 VALU instructions, against 13 for dequantising to scaled fp16 weights.
//
// Work split: NT tiles of 16 channels per workgroup and NWT waves per tile; wave part q of
// the tile owns groups [gs0 + q gpw, gs0 + (q+1) gpw) of the workgroup's K range (gpw a
// multiple of 8).  Parts past the end of K run on clamped addresses and add nothing.  The
// activations are staged into LDS in chunks of CG groups per part (double-buffered, one
// LDS-only barrier per chunk, rows swizzled as in the other kernels); the weights stream
// through a P-group register ring; scales and zeros come as 8-group vectors.  The NWT part
// sums of a tile are added through LDS in part order; with splits > 1 the split sums go
// through the workspace and the last workgroup of the tile block adds them in split order, so
// results are bitwise reproducible.
template <int MV, int NT, int NWT, int P, int CG, bool FOLD>
__global__ __launch_bounds__(NT * NWT * 64) void w4a16_small_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, unsigned* __restrict__ counters, float* __restrict__ part,
    int splits, int gpw, int reduce_launch) {
  static_assert(8 % P == 0 && 8 % CG == 0, "P and CG divide the 8-group body");
  static_assert(MV == 1 || MV == 2 || MV == 4, "outputs per lane");
  constexpr int NW = NT * NWT;
  constexpr int NTHR = NW * 64;
  constexpr int VG = CG * 16;             // 16-byte vectors per token row per part per chunk
  constexpr int VC = NWT * VG;            // per token row per chunk (a power of two)
  constexpr int ROWS = MV < 4 ? MV : 16;  // the most token rows a launch of this MV holds
  constexpr int XV = (ROWS * VC + NTHR - 1) / NTHR;  // staged vectors per thread
  extern __shared__ u32x4 xs[];  // [2][M][VC] + 1 spare vector; afterwards the part sums
  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3, G = K >> 7;
  const int wpart = wave % NWT;
  const int tile = blockIdx.x * NT + wave / NWT;
  const bool tv = tile * 16 < N;
  const int n = (tv ? tile * 16 : 0) + r;
  const int gs0 = blockIdx.y * NWT * gpw;  // the workgroup's first group
  const int gw0 = gs0 + wpart * gpw;       // this wave's first group
  // Groups of this wave inside K (a multiple of 8, possibly 0), and the last group index its
  // loads may use: addresses are based at a group that exists (G >= 8 is a host rule).
  const int nvalid = max(0, min(gpw, G - gw0));
  const int gwa = min(gw0, G - 8);
  const int glast = max(nvalid, 8) - 1;
  const int nch = gpw / CG;

  const uint32_t* wrow = qw + (size_t)n * KW + (size_t)gwa * 16 + kg * 4;
  const uint16_t* srow = scales + (size_t)n * G + gwa;
  const uint8_t* zrow = zeros + (size_t)n * G + gwa;

  u32x4 wq[P];
  u32x4 s_cur, s_nxt;
  u32x2 z_cur, z_nxt;
  auto load_w = [&](int g, int slot) {
    wq[slot] = *reinterpret_cast<const u32x4*>(wrow + (size_t)min(g, glast) * 16);
  };
  auto load_blk = [&](int g) {  // g: a multiple of 8
    const int gb = min(g, glast - 7);
    s_nxt = *reinterpret_cast<const u32x4*>(srow + gb);
    z_nxt = *reinterpret_cast<const u32x2*>(zrow + gb);
  };

  // Chunk staging: thread tid owns vectors e = tid + j NTHR of the M x VC chunk (row m = e /
  // VC, vector v = e % VC of part v / VG).  Rows past M load row M - 1 and store to the spare
  // vector after both buffers (the stores stay unconditional, see w4a16_chunk_kernel); a
  // column past K (a part beyond the end) reads the row's last vector.
  uint32_t roff[XV], koff[XV];
  int loff[XV], lstep[XV];
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int e = tid + j * NTHR;
    const int m = e / VC, v = e % VC;
    roff[j] = (uint32_t)min(m, M - 1) * (uint32_t)K;
    koff[j] = (uint32_t)((v / VG) * gpw * 128 + (v % VG) * 8);
    loff[j] = m < M ? m * VC + swz(m, v) : 2 * M * VC;
    lstep[j] = m < M ? M * VC : 0;
  }
  u32x4 xr[XV];
  auto load_chunk = [&](int c) {
    const uint32_t kb = (uint32_t)(gs0 + c * CG) * 128u;
#pragma unroll
    for (int j = 0; j < XV; ++j)
      xr[j] = *reinterpret_cast<const u32x4*>(x + roff[j] + min(kb + koff[j], (uint32_t)K - 8u));
  };
  auto store_chunk = [&](int c) {
#pragma unroll
    for (int j = 0; j < XV; ++j) xs[loff[j] + (c & 1) * lstep[j]] = permute_x(xr[j]);
  };

  load_blk(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_w(p, p);
  __builtin_amdgcn_sched_barrier(0);
  load_chunk(0);
  store_chunk(0);
  load_chunk(min(1, nch - 1));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // LDS vector of this lane's A fragment for K-step i of chunk-group j in buffer b:
  // aoff[i] + 16 j + b M VC (token rows past M read row M - 1; their sums are not stored).
  const int mr = min(r, M - 1);
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = mr * VC + wpart * VG + swz(mr, kg * 4 + i);

  float acc[MV];
#pragma unroll
  for (int v = 0; v < MV; ++v) acc[v] = 0.f;

  auto body = [&](int gb) {
    s_cur = s_nxt;
    z_cur = z_nxt;
    const bool valid = gb < nvalid;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int g = gb + p;
      const int slot = p % P;
      // The scale's half of its word by shift and mask (taking an element of an fp16 pair
      // bit-cast from a vector component was miscompiled to component 0 here).
      const uint32_t sw = s_cur[p >> 1];
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)((p & 1) ? sw >> 16 : sw & 0xFFFFu));
      const uint32_t zz = zero_pair(z_cur, p);
      // FOLD: -(1024 + z), -(64 + z); else (1024 + z), (64 + z); pairs in dequant order.
      const uint32_t zl = zz | (FOLD ? 0xE400E400u : 0x64006400u);
      const uint32_t zh = (zz << 4) | (FOLD ? 0xD400D400u : 0x54005400u);
      if (p == 8 - P) {  // the next body's scales and zeros
        load_blk(gb + 8);
        __builtin_amdgcn_sched_barrier(0);
      }
      const u32x4* buf = xs + ((g / CG) & 1) * (M * VC) + (p % CG) * 16;
      f32x4 gs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x8 a = __builtin_bit_cast(f16x8, buf[aoff[i]]);
        if (FOLD) {
          const u32x4 u = unpack8(wq[slot][i], uk);
          gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, u), gs, 0, 0, 0);
          gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a, __builtin_bit_cast(f16x8, u32x4{zl, zh, zl, zh}), gs, 0, 0, 0);
        } else {
          const u32x4 b = unpack8_minus_zero(wq[slot][i], zl, zh, uk);
          gs = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, b), gs, 0, 0, 0);
        }
      }
      load_w(g + P, slot);  // the slot's words are all unpacked
      __builtin_amdgcn_sched_barrier(0);
      if (valid) {
#pragma unroll
        for (int v = 0; v < MV; ++v) acc[v] = __builtin_fmaf(s, gs[v], acc[v]);
      }
      if (p % CG == CG - 1) {  // end of chunk g / CG: stage the one after next
        const int c = g / CG;
        store_chunk(c + 1);
        load_chunk(min(c + 2, nch - 1));
        lds_barrier();
      }
    }
  };
  body(0);
  for (int gb = 8; gb < gpw; gb += 8) body(gb);

  // Part sums of each tile, in part order (every wave is past the last chunk barrier, so the
  // staged activations are dead).
  if (NWT > 1) {
    float* red = reinterpret_cast<float*>(xs);
#pragma unroll
    for (int v = 0; v < MV; ++v) red[(wave * MV + v) * 64 + lane] = acc[v];
    __syncthreads();
    if (wpart == 0) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        float t = red[(wave * MV + v) * 64 + lane];
#pragma unroll
        for (int q = 1; q < NWT; ++q) t += red[((wave + q) * MV + v) * 64 + lane];
        acc[v] = t;
      }
    }
  }

  // Lane (r, kg) holds tokens 4 kg + v of channel n.
  if (splits == 1) {
    if (wpart == 0 && tv) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        const int m = kg * 4 + v;
        if (m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[v]);
      }
    }
    return;
  }
  if (reduce_launch) {  // a second launch adds the splits: plain stores, nothing to wait for
    if (wpart == 0 && tv) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        const int m = kg * 4 + v;
        if (m < M) part[((size_t)blockIdx.y * M + m) * N + n] = acc[v];
      }
    }
    return;
  }
  if (wpart == 0 && tv) {
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      const int m = kg * 4 + v;
      if (m < M) st_coherent(&part[((size_t)blockIdx.y * M + m) * N + n], acc[v]);
    }
  }
  if (!arrive_last(&counters[blockIdx.x], (unsigned)splits)) return;
  for (int t = tid; t < NT * 16 * M; t += NTHR) {
    const int tt = t / (16 * M), rem = t - tt * 16 * M;
    const int m = rem >> 4;
    const int nn = (blockIdx.x * NT + tt) * 16 + (rem & 15);
    if (nn >= N) continue;
    float sum = 0.f;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      float v8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v8[j] = ld_coherent(&part[((size_t)min(sp0 + j, splits - 1) * M + m) * N + nn]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (sp0 + j < splits) sum += v8[j];
    }
    y[(size_t)m * N + nn] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// W4A16 for one token tile (M <= 16) with the workgroup's whole K range staged once.
//
// Same arithmetic as w4a16_small_kernel (activations as the MFMA's A operand, fp32 group sums
// scaled per group, offsets and zero points removed exactly), but the main loop's only
// global loads are the weight ring: before it, the workgroup stages in one round of
// cooperative, coalesced loads (a) its whole activation slice, M rows x NWT gpw groups,
// permuted and swizzled as in the other kernels, and (b) the scale and zero point of
// every (channel, group) it covers, packed as scale | zero << 16 in one 32-bit word, stored
// [group][channel] so that a wave's 16 channels read 16 consecutive words.  One barrier, then
// every wave streams its weights through a P-group register ring with no barrier and no other
// global load (a per-group scale/zero load in the weight stream, or activation loads between
// weight loads, measured 5-10 % of the launch each).  The host sizes the K split so that the
// staged slice fits in LDS.
template <int MV, int NT, int NWT, int P, bool FOLD>
__global__ __launch_bounds__(NT * NWT * 64) void w4a16_slice_kernel(
    const uint16_t* __restrict__ x, int M, int K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int N,
    uint16_t* __restrict__ y, unsigned* __restrict__ counters, float* __restrict__ part,
    int splits, int gpw, int reduce_launch) {
  static_assert(8 % P == 0, "P divides the 8-group body");
  static_assert(MV == 1 || MV == 2 || MV == 4, "outputs per lane");
  constexpr int NW = NT * NWT;
  constexpr int NTHR = NW * 64;
  constexpr int NCH = NT * 16;            // channels per workgroup
  extern __shared__ u32x4 xs[];           // [M][VW] activations, then [GW][NCH] scale|zero words
  const UnpackK uk = unpack_consts();
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, r = lane & 15, kg = lane >> 4;
  const int KW = K >> 3, G = K >> 7;
  const int wpart = wave % NWT;
  const int tloc = wave / NWT;
  const int tile = blockIdx.x * NT + tloc;
  const bool tv = tile * 16 < N;
  const int n = (tv ? tile * 16 : 0) + r;
  const int GW = NWT * gpw;               // groups of the workgroup
  const int VW = GW * 16;                 // 16-byte activation vectors per staged row
  const int gs0 = blockIdx.y * GW;
  const int gw0 = gs0 + wpart * gpw;
  const int nvalid = max(0, min(gpw, G - gw0));
  const int gwa = min(gw0, G - 8);
  const int glast = max(nvalid, 8) - 1;
  uint32_t* szs = reinterpret_cast<uint32_t*>(xs + M * VW);

  const uint32_t* wrow = qw + (size_t)n * KW + (size_t)gwa * 16 + kg * 4;
  u32x4 wq[P];
  auto load_w = [&](int g, int slot) {
    wq[slot] = *reinterpret_cast<const u32x4*>(wrow + (size_t)min(g, glast) * 16);
  };

  // Staging loads first (they hit in L2), then the weight ring: loads return in order, so the
  // LDS stores below wait for the staging loads only and the ring stays in flight across the
  // barrier.  Activations: vector e of the M x VW slice (row e / VW); columns past K (a part
  // beyond the end) read the row's last vector.  Up to XS vectors per thread go through
  // registers in this first pass; a larger slice (many tokens) stages the rest afterwards.
  constexpr int XS = 4;
  const int nvec = M * VW;
  u32x4 d[XS];
  int ea[XS];
#pragma unroll
  for (int j = 0; j < XS; ++j) {
    const int e = min(tid + j * NTHR, nvec - 1);
    const int m = e / VW, v = e - m * VW;
    const int k = min((gs0 + (v >> 4)) * 128 + (v & 15) * 8, K - 8);
    d[j] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k);
    ea[j] = tid + j * NTHR < nvec ? m * VW + swz(m, v) : -1;
  }
  // Scale | zero << 16 for (channel c, group g) go to szs[g * NCH + c]: thread t takes the
  // 8-group block t / NCH of channel t % NCH (16 + 8 bytes, one load each).
  const int nblk = NCH * (GW / 8);
  u32x4 sv;
  u32x2 zv;
  int sc = -1, sb = 0;
  if (tid < nblk) {
    sc = tid % NCH;
    sb = tid / NCH;
    const int nc = min((blockIdx.x * NT) * 16 + sc, N - 1);
    const int gb = min(gs0 + sb * 8, G - 8);
    sv = *reinterpret_cast<const u32x4*>(scales + (size_t)nc * G + gb);
    zv = *reinterpret_cast<const u32x2*>(zeros + (size_t)nc * G + gb);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < P; ++p) load_w(p, p);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < XS; ++j)
    if (ea[j] >= 0) xs[ea[j]] = permute_x(d[j]);
  auto store_sz = [&](int c, int b, const u32x4& svv, const u32x2& zvv) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sh = (svv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
      const uint32_t zb = (zvv[j >> 2] >> (8 * (j & 3))) & 0xFFu;
      szs[(b * 8 + j) * NCH + c] = sh | (zb << 16);
    }
  };
  if (sc >= 0) store_sz(sc, sb, sv, zv);
  // The rest of a large slice (more than XS vectors per thread, or more 8-group blocks than
  // threads).  From two tokens on: staging rounds of XS loads, then XS stores; vectors past
  // the slice's end load and store a copy of its last one, to its own place (identical
  // values): a plain loop waits for each load alone, one L2 round trip per vector.  (One
  // token keeps the plain loop, which its usual slices never reach, and the registers.)
  if constexpr (MV == 1) {
    for (int e = tid + XS * NTHR; e < nvec; e += NTHR) {
      const int m = e / VW, v = e - m * VW;
      const int k = min((gs0 + (v >> 4)) * 128 + (v & 15) * 8, K - 8);
      xs[m * VW + swz(m, v)] = permute_x(*reinterpret_cast<const u32x4*>(x + (size_t)m * K + k));
    }
  } else {
  for (int e0 = tid + XS * NTHR; e0 < nvec; e0 += XS * NTHR) {
    u32x4 dd[XS];
    int ee[XS];
#pragma unroll
    for (int j = 0; j < XS; ++j) {
      const int e = min(e0 + j * NTHR, nvec - 1);
      const int m = e / VW, v = e - m * VW;
      const int k = min((gs0 + (v >> 4)) * 128 + (v & 15) * 8, K - 8);
      dd[j] = *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k);
      ee[j] = m * VW + swz(m, v);
    }
#pragma unroll
    for (int j = 0; j < XS; ++j) xs[ee[j]] = permute_x(dd[j]);
  }
  }
  for (int t = tid + NTHR; t < nblk; t += NTHR) {
    const int c = t % NCH, b = t / NCH;
    const int nc = min((blockIdx.x * NT) * 16 + c, N - 1);
    const int gb = min(gs0 + b * 8, G - 8);
    store_sz(c, b, *reinterpret_cast<const u32x4*>(scales + (size_t)nc * G + gb),
             *reinterpret_cast<const u32x2*>(zeros + (size_t)nc * G + gb));
  }
  __syncthreads();

  const int mr = min(r, M - 1);
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = mr * VW + wpart * gpw * 16 + swz(mr, kg * 4 + i);
  const uint32_t* szw = szs + (wpart * gpw) * NCH + tloc * 16 + r;  // this lane's channel

  float acc[MV];
#pragma unroll
  for (int v = 0; v < MV; ++v) acc[v] = 0.f;

  for (int gb = 0; gb < gpw; gb += 8) {
    const bool valid = gb < nvalid;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int g = gb + p;
      const int slot = p % P;
      const uint32_t sz = szw[g * NCH];
      // (1024 + z, 64 + z) pairs, negated for FOLD; z sits in byte 2 of sz.
      const uint32_t zz = __builtin_amdgcn_perm(0u, sz, 0x0C020C02u);
      const uint32_t zl = zz | (FOLD ? 0xE400E400u : 0x64006400u);
      const uint32_t zh = (zz << 4) | (FOLD ? 0xD400D400u : 0x54005400u);
      const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(sz & 0xFFFFu));
      const u32x4* buf = xs + g * 16;
      f32x4 gsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f16x8 a = __builtin_bit_cast(f16x8, buf[aoff[i]]);
        if (FOLD) {
          const u32x4 u = unpack8(wq[slot][i], uk);
          gsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, u), gsum, 0, 0, 0);
          gsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a, __builtin_bit_cast(f16x8, u32x4{zl, zh, zl, zh}), gsum, 0, 0, 0);
        } else {
          const u32x4 b = unpack8_minus_zero(wq[slot][i], zl, zh, uk);
          gsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, b), gsum, 0, 0, 0);
        }
      }
      load_w(g + P, slot);  // the slot's words are all unpacked
      __builtin_amdgcn_sched_barrier(0);
      if (valid) {
#pragma unroll
        for (int v = 0; v < MV; ++v) acc[v] = __builtin_fmaf(s, gsum[v], acc[v]);
      }
    }
  }

  if (NWT > 1) {
    __syncthreads();  // every wave is done with the staged slice
    float* red = reinterpret_cast<float*>(xs);
#pragma unroll
    for (int v = 0; v < MV; ++v) red[(wave * MV + v) * 64 + lane] = acc[v];
    __syncthreads();
    if (wpart == 0) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        float t = red[(wave * MV + v) * 64 + lane];
#pragma unroll
        for (int q = 1; q < NWT; ++q) t += red[((wave + q) * MV + v) * 64 + lane];
        acc[v] = t;
      }
    }
  }

  if (splits == 1) {
    if (wpart == 0 && tv) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        const int m = kg * 4 + v;
        if (m < M) y[(size_t)m * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[v]);
      }
    }
    return;
  }
  if (reduce_launch) {  // a second launch adds the splits: plain stores, nothing to wait for
    if (wpart == 0 && tv) {
#pragma unroll
      for (int v = 0; v < MV; ++v) {
        const int m = kg * 4 + v;
        if (m < M) part[((size_t)blockIdx.y * M + m) * N + n] = acc[v];
      }
    }
    return;
  }
  if (wpart == 0 && tv) {
#pragma unroll
    for (int v = 0; v < MV; ++v) {
      const int m = kg * 4 + v;
      if (m < M) st_coherent(&part[((size_t)blockIdx.y * M + m) * N + n], acc[v]);
    }
  }
  if (!arrive_last(&counters[blockIdx.x], (unsigned)splits)) return;
  for (int t = tid; t < NCH * M; t += NTHR) {
    const int tt = t / (16 * M), rem = t - tt * 16 * M;
    const int m = rem >> 4;
    const int nn = (blockIdx.x * NT + tt) * 16 + (rem & 15);
    if (nn >= N) continue;
    float sum = 0.f;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      float v8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v8[j] = ld_coherent(&part[((size_t)min(sp0 + j, splits - 1) * M + m) * N + nn]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (sp0 + j < splits) sum += v8[j];
    }
    y[(size_t)m * N + nn] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

constexpr int kNW = 4;
constexpr int kNT = 2;
constexpr int kCG = 2;

template <int MT>
hipError_t launch_staged(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                         const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                         unsigned* counters, void* partials, hipStream_t stream) {
  dim3 grid(p.tiles, p.splits);
  w4a16_kernel<MT, kNT, kNW, kCG><<<grid, kNW * 64, 0, stream>>>(
      x, M, K, qw, scales, zeros, N, y, counters, static_cast<float*>(partials), p.splits,
      p.k_per_split);
  return hipGetLastError();
}

// Ring configurations: (NT tiles per wave, NW waves per workgroup, P groups in flight).
struct RingCfg { int nt, nw, p; };
constexpr RingCfg kRing[] = {{0, 0, 0}, {2, 8, 4}, {1, 8, 4}, {2, 4, 4}, {1, 8, 8}, {2, 8, 2}};
constexpr int kNumRing = sizeof(kRing) / sizeof(kRing[0]);
constexpr size_t kRingLdsMax = 156 * 1024;  // leaves room for static LDS

template <int MT, int C>
hipError_t launch_ring(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                       const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                       unsigned* counters, void* partials, hipStream_t stream) {
  constexpr RingCfg c = kRing[C];
  const int gps = p.k_per_split / 128;
  const size_t lds = (size_t)M * gps * 16 * sizeof(u32x4);
  // Vector scale/zero loads need 8-group rows and slices and aligned arrays.
  const bool vec = (K / 128) % 8 == 0 && gps % 8 == 0 && ((uintptr_t)scales % 16) == 0 &&
                   ((uintptr_t)zeros % 8) == 0;
  auto kern = vec ? w4a16_ring_kernel<MT, c.nt, c.nw, c.p, true>
                  : w4a16_ring_kernel<MT, c.nt, c.nw, c.p, false>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles, p.splits);
  kern<<<grid, c.nw * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y, counters,
                                        static_cast<float*>(partials), p.splits, gps);
  return hipGetLastError();
}

// Chunked configurations: (NT, NW, P, CG).
struct ChunkShape { int nt, nw, p, cg; };
constexpr ChunkShape kChunkShapes[] = {{1, 8, 4, 4}, {2, 8, 2, 4}, {1, 16, 4, 4}, {2, 8, 4, 4},
                                       {1, 8, 2, 2}, {1, 8, 8, 4}, {1, 16, 8, 4}, {1, 8, 8, 2},
                                       {2, 7, 4, 4}, {1, 10, 2, 2}};
constexpr int kNumChunkShapes = sizeof(kChunkShapes) / sizeof(kChunkShapes[0]);
constexpr int kChunkBase = 10;  // configuration indices kChunkBase + i
constexpr int kStagedCfg = 9;   // the LDS-staged kernel (w4a16_kernel)

size_t chunk_lds_bytes(int M, int cg) {
  const size_t rows = (size_t)(M + 15) / 16 * 16;  // padded to whole token tiles
  return ((size_t)2 * rows * cg * 16 + 1) * sizeof(u32x4);
}

template <int MT, int I>
hipError_t launch_chunk(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream) {
  constexpr ChunkShape c = kChunkShapes[I];
  // Every split must hold a multiple of 8 groups (the kernel's loop body has no exits) and
  // scales/zeros must allow 8-group vector loads.
  const int gps = p.k_per_split / 128;
  if ((K / 128) % 8 != 0 || gps % 8 != 0 || ((uintptr_t)scales % 16) != 0 ||
      ((uintptr_t)zeros % 8) != 0)
    return hipErrorInvalidValue;
  const size_t lds = chunk_lds_bytes(M, c.cg);
  auto kern = w4a16_chunk_kernel<MT, c.nt, c.nw, c.p, c.cg>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles, p.splits);
  const bool red = p.splits > 1 && p.reduce_launch;
  kern<<<grid, c.nw * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y, counters,
                                        static_cast<float*>(partials), p.splits, gps, red ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !red) return e;
  return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, nullptr, y,
                              stream);
}

// Configurations of the kernel with a staging wave: (NT tiles per compute wave, NW compute
// waves, P groups in flight, CG groups per chunk).  Index kStageBase + i.  One staging wave
// holds a whole chunk (16 MT x 16 CG vectors over 64 lanes, at most 48 per lane).
struct StageShape { int nt, nw, p, cg; };
constexpr StageShape kStageShapes[] = {{2, 7, 4, 4}, {2, 7, 2, 4}, {2, 7, 4, 2}, {1, 7, 4, 2}};
constexpr int kNumStageShapes = sizeof(kStageShapes) / sizeof(kStageShapes[0]);
constexpr int kStageBase = 110;

bool stage_fits(int M, int cg) { return (M + 15) / 16 * cg * 4 <= 48; }

template <int MT, int I>
hipError_t launch_stage_t(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                          void* partials, hipStream_t stream) {
  constexpr StageShape c = kStageShapes[I];
  const int gps = p.k_per_split / 128;
  if ((K / 128) % 8 != 0 || gps % 8 != 0 || ((uintptr_t)scales % 16) != 0 ||
      ((uintptr_t)zeros % 8) != 0 || (M + 15) / 16 != MT || (p.splits > 1 && !partials))
    return hipErrorInvalidValue;
  if constexpr (MT * c.cg * 4 > 48) {
    return hipErrorInvalidValue;
  } else {
    const size_t lds = chunk_lds_bytes(M, c.cg);
    auto kern = w4a16_stage_kernel<MT, c.nt, c.nw, c.p, c.cg>;
    if (lds > 64 * 1024) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    dim3 grid(p.tiles, p.splits);
    kern<<<grid, (c.nw + 1) * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y,
                                                 static_cast<float*>(partials), p.splits, gps);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, nullptr, y,
                                stream);
  }
}

template <int MT>
hipError_t launch_stage_mt(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                           const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                           void* partials, hipStream_t stream) {
  switch (p.waves - kStageBase) {
#define QV_STAGE(I) \
  case I: return launch_stage_t<MT, I>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    QV_STAGE(0) QV_STAGE(1) QV_STAGE(2) QV_STAGE(3)
#undef QV_STAGE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stage(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        void* partials, hipStream_t stream) {
  switch ((M + 15) / 16) {
    case 1: return launch_stage_mt<1>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    case 2: return launch_stage_mt<2>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    case 3: return launch_stage_mt<3>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    case 4: return launch_stage_mt<4>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

// Wide configurations (32x32x16 MFMAs): (NT 32-channel tiles per wave, NW waves, P groups in
// flight, CG groups per chunk).  Index kWideBase + i.
struct WideShape { int nt, nw, p, cg; };
constexpr WideShape kWideShapes[] = {{1, 8, 2, 2}, {1, 8, 4, 2}, {1, 4, 4, 2}, {2, 4, 2, 2}};
constexpr int kNumWideShapes = sizeof(kWideShapes) / sizeof(kWideShapes[0]);
constexpr int kWideBase = 100;

size_t wide_lds_bytes(int M, int cg) {
  const size_t rows = (size_t)(M + 31) / 32 * 32;
  return ((size_t)2 * rows * cg * 16 + 1) * sizeof(u32x4);
}

template <int MT, int I>
hipError_t launch_wide_t(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                         const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                         void* partials, hipStream_t stream) {
  constexpr WideShape c = kWideShapes[I];
  const int gps = p.k_per_split / 128;
  if ((K / 128) % 8 != 0 || gps % 8 != 0 || ((uintptr_t)scales % 16) != 0 ||
      ((uintptr_t)zeros % 8) != 0 || (M + 31) / 32 != MT || (p.splits > 1 && !partials))
    return hipErrorInvalidValue;
  const size_t lds = wide_lds_bytes(M, c.cg);
  auto kern = w4a16_wide_kernel<MT, c.nt, c.nw, c.p, c.cg>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles, p.splits);
  kern<<<grid, c.nw * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y,
                                        static_cast<float*>(partials), p.splits, gps);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, nullptr, y,
                              stream);
}

template <int MT>
hipError_t launch_wide_mt(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                          void* partials, hipStream_t stream) {
  switch (p.waves - kWideBase) {
#define QV_WIDE(I) \
  case I: return launch_wide_t<MT, I>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
    QV_WIDE(0) QV_WIDE(1) QV_WIDE(2) QV_WIDE(3)
#undef QV_WIDE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wide(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                       const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                       void* partials, hipStream_t stream) {
  if (M <= 32) return launch_wide_mt<1>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
  return launch_wide_mt<2>(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
}

// Small-M configurations: (NT tiles per workgroup, NWT waves per tile, P groups in flight,
// CG groups per staged chunk).  Index kSmallBase + i, or kSmallBase + kFoldOffset + i for the
// zero-point-MFMA form.
struct SmallShape { int nt, nwt, p, cg; };
constexpr SmallShape kSmallShapes[] = {{8, 1, 4, 8}, {2, 4, 4, 4}, {4, 2, 4, 4},
                                       {8, 1, 8, 8}, {2, 4, 8, 4}, {2, 4, 4, 2}};
constexpr int kNumSmallShapes = sizeof(kSmallShapes) / sizeof(kSmallShapes[0]);
constexpr int kSmallBase = 20;
constexpr int kFoldOffset = 20;
constexpr size_t kSmallLdsMax = 156 * 1024;

size_t small_lds_bytes(int M, int mv, const SmallShape& c) {
  const size_t xsb = ((size_t)2 * M * c.nwt * c.cg * 16 + 1) * sizeof(u32x4);
  const size_t red = c.nwt > 1 ? (size_t)c.nt * c.nwt * mv * 64 * sizeof(float) : 0;
  return xsb > red ? xsb : red;
}

int small_mv(int M) { return M <= 2 ? M : 4; }

template <int MV, int I, bool FOLD>
hipError_t launch_small_t(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                          unsigned* counters, void* partials, hipStream_t stream) {
  constexpr SmallShape c = kSmallShapes[I];
  const int gpw = p.k_per_split / 128;  // groups per wave
  // The kernel's preconditions: 8-group scale/zero vectors (aligned arrays, whole blocks),
  // every wave range a multiple of 8 groups, every tile block and K range covered.
  if ((K / 128) % 8 != 0 || gpw % 8 != 0 || gpw < 8 || ((uintptr_t)scales % 16) != 0 ||
      ((uintptr_t)zeros % 8) != 0 || M > (MV < 4 ? MV : 16) ||
      (long long)p.tiles * c.nt * 16 < N || (long long)p.splits * c.nwt * gpw < K / 128)
    return hipErrorInvalidValue;
  const size_t lds = small_lds_bytes(M, MV, c);
  auto kern = w4a16_small_kernel<MV, c.nt, c.nwt, c.p, c.cg, FOLD>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles, p.splits);
  const bool red = p.splits > 1 && p.reduce_launch;
  kern<<<grid, c.nt * c.nwt * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y, counters,
                                                static_cast<float*>(partials), p.splits, gpw,
                                                red ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !red) return e;
  return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, nullptr, y,
                              stream);
}

template <int MV, bool FOLD>
hipError_t launch_small_f(int i, const GemmPlan& p, const uint16_t* x, int M, int K,
                          const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                          uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
#define QV_SMALL(I) \
  case I: return launch_small_t<MV, I, FOLD>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  switch (i) {
    QV_SMALL(0) QV_SMALL(1) QV_SMALL(2) QV_SMALL(3) QV_SMALL(4) QV_SMALL(5)
    default: return hipErrorInvalidValue;
  }
#undef QV_SMALL
}

hipError_t launch_small(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream) {
  const bool fold = p.waves >= kSmallBase + kFoldOffset;
  const int i = p.waves - kSmallBase - (fold ? kFoldOffset : 0);
  const int mv = small_mv(M);
#define QV_SMALL_MV(MV)                                                                            \
  if (mv == MV)                                                                                  \
    return fold ? launch_small_f<MV, true>(i, p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream) \
                : launch_small_f<MV, false>(i, p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  QV_SMALL_MV(1)
  QV_SMALL_MV(2)
  QV_SMALL_MV(4)
#undef QV_SMALL_MV
  return hipErrorInvalidValue;
}

// Whole-slice configurations: (NT tiles per workgroup, NWT waves per tile, P groups in
// flight).  Index kSliceBase + i, or kSliceBase + kFoldOffset + i for the zero-point-MFMA form.
struct SliceShape { int nt, nwt, p; };
constexpr SliceShape kSliceShapes[] = {{4, 2, 4}, {2, 4, 4}, {8, 1, 4}, {1, 8, 4},
                                       {4, 2, 8}, {2, 4, 8}, {1, 8, 8}, {2, 2, 4}};
constexpr int kNumSliceShapes = sizeof(kSliceShapes) / sizeof(kSliceShapes[0]);
constexpr int kSliceBase = 60;
constexpr size_t kSliceLdsTarget = 64 * 1024;  // two or more workgroups per CU

size_t slice_lds_bytes(int M, int mv, const SliceShape& c, int gw) {
  const size_t xsb = (size_t)M * gw * 16 * sizeof(u32x4) + (size_t)gw * c.nt * 16 * sizeof(uint32_t);
  const size_t red = c.nwt > 1 ? (size_t)c.nt * c.nwt * mv * 64 * sizeof(float) : 0;
  return xsb > red ? xsb : red;
}

template <int MV, int I, bool FOLD>
hipError_t launch_slice_t(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                          unsigned* counters, void* partials, hipStream_t stream) {
  constexpr SliceShape c = kSliceShapes[I];
  const int gpw = p.k_per_split / 128;  // groups per wave
  if ((K / 128) % 8 != 0 || gpw % 8 != 0 || gpw < 8 || ((uintptr_t)scales % 16) != 0 ||
      ((uintptr_t)zeros % 8) != 0 || M > (MV < 4 ? MV : 16) ||
      (long long)p.tiles * c.nt * 16 < N || (long long)p.splits * c.nwt * gpw < K / 128)
    return hipErrorInvalidValue;
  const size_t lds = slice_lds_bytes(M, MV, c, c.nwt * gpw);
  if (lds > kSmallLdsMax) return hipErrorInvalidValue;
  auto kern = w4a16_slice_kernel<MV, c.nt, c.nwt, c.p, FOLD>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles, p.splits);
  const bool red = p.splits > 1 && p.reduce_launch;
  kern<<<grid, c.nt * c.nwt * 64, lds, stream>>>(x, M, K, qw, scales, zeros, N, y, counters,
                                                static_cast<float*>(partials), p.splits, gpw,
                                                red ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !red) return e;
  return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, nullptr, y,
                              stream);
}

template <int MV, bool FOLD>
hipError_t launch_slice_f(int i, const GemmPlan& p, const uint16_t* x, int M, int K,
                          const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                          uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
#define QV_SLICE(I) \
  case I: return launch_slice_t<MV, I, FOLD>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  switch (i) {
    QV_SLICE(0) QV_SLICE(1) QV_SLICE(2) QV_SLICE(3) QV_SLICE(4) QV_SLICE(5) QV_SLICE(6) QV_SLICE(7)
    default: return hipErrorInvalidValue;
  }
#undef QV_SLICE
}

hipError_t launch_slice(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream) {
  const bool fold = p.waves >= kSliceBase + kFoldOffset;
  const int i = p.waves - kSliceBase - (fold ? kFoldOffset : 0);
  const int mv = small_mv(M);
#define QV_SLICE_MV(MV)                                                                            \
  if (mv == MV)                                                                                  \
    return fold ? launch_slice_f<MV, true>(i, p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream) \
                : launch_slice_f<MV, false>(i, p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  QV_SLICE_MV(1)
  QV_SLICE_MV(2)
  QV_SLICE_MV(4)
#undef QV_SLICE_MV
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_mt(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                     const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                     unsigned* counters, void* partials, hipStream_t stream) {
  switch (p.waves) {  // `waves` carries the configuration index here
    case 1: return launch_ring<MT, 1>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 2: return launch_ring<MT, 2>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 3: return launch_ring<MT, 3>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 4: return launch_ring<MT, 4>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 5: return launch_ring<MT, 5>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 0: return launch_chunk<MT, 0>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 1: return launch_chunk<MT, 1>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 2: return launch_chunk<MT, 2>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 3: return launch_chunk<MT, 3>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 4: return launch_chunk<MT, 4>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 5: return launch_chunk<MT, 5>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 6: return launch_chunk<MT, 6>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 7: return launch_chunk<MT, 7>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 8: return launch_chunk<MT, 8>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kChunkBase + 9: return launch_chunk<MT, 9>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case kStagedCfg: return launch_staged<MT>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace {

// Plan of the small-M kernel, configuration index cfg (kSmallBase + i [+ kFoldOffset]).
GemmPlan plan_small(int M, int N, int K, int cfg, const Tuning& t) {
  GemmPlan p{};
  const int i = cfg - kSmallBase - (cfg >= kSmallBase + kFoldOffset ? kFoldOffset : 0);
  const SmallShape c = kSmallShapes[i];
  const int blocks = K / 1024;  // 8-group blocks
  p.waves = cfg;
  p.tiles = (N + 16 * c.nt - 1) / (16 * c.nt);
  // K is split across workgroups only until the launch has about 2048 waves (8 per CU).
  const int waves1 = (N / 16) * c.nwt;
  int splits = waves1 < 2048 ? (2048 + waves1 - 1) / waves1 : 1;
  if (int e = t(QV_TUNE_W4A16_SPLITS)) splits = e;
  if (splits < 1) splits = 1;
  // Groups per wave: whole 8-group blocks covering K with NWT parts per split.
  int bpw = (blocks + c.nwt * splits - 1) / (c.nwt * splits);
  if (bpw < 1) bpw = 1;
  splits = (blocks + c.nwt * bpw - 1) / (c.nwt * bpw);
  p.splits = splits;
  p.k_per_split = bpw * 8 * 128;
  p.variant = 1;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  p.reduce_launch = t(QV_TUNE_W4A16_REDUCE) == 2;
  p.ok = small_lds_bytes(M, small_mv(M), c) <= kSmallLdsMax &&
         (splits == 1 || p.tiles <= (int)(QV_WORKSPACE_COUNTER_BYTES / 4));
  return p;
}

// Plan of the whole-slice kernel, configuration index cfg (kSliceBase + i [+ kFoldOffset]).
GemmPlan plan_slice(int M, int N, int K, int cfg, const Tuning& t) {
  GemmPlan p{};
  const int i = cfg - kSliceBase - (cfg >= kSliceBase + kFoldOffset ? kFoldOffset : 0);
  const SliceShape c = kSliceShapes[i];
  const int blocks = K / 1024;  // 8-group blocks
  const int mv = small_mv(M);
  p.waves = cfg;
  p.tiles = (N + 16 * c.nt - 1) / (16 * c.nt);
  // K is split across workgroups only until the launch has about 1024 waves (measured on the
  // Llama-3-70B linears at M = 1: fewer, longer waves beat more, shorter ones, which pay the
  // staging prologue and the ring's ramp more often: qkv 14.2 -> 12.7 us, o 12.4 -> 9.7 us,
  // down 29.7 -> 26.6 us with one split instead of two), and further while the staged slice
  // exceeds 64 KB of LDS (so that several workgroups share a CU).
  const int waves1 = (N / 16) * c.nwt;
  int splits = waves1 < 1024 ? (1024 + waves1 - 1) / waves1 : 1;
  const int forced = t(QV_TUNE_W4A16_SPLITS);
  if (forced) splits = forced;
  if (splits < 1) splits = 1;
  // Blocks per wave for `splits` splits: the K range spread as evenly as whole 8-group blocks
  // allow.  Past the LDS target, add splits (not drop blocks from the first splits only,
  // which leaves the last split with the remainder: the down projection at M = 1 had waves of
  // 5 and 2 blocks instead of 4 and 3, qkv at M = 4 splits of 48 and 16 groups).
  auto per_wave = [&](int s) {
    const int b = (blocks + c.nwt * s - 1) / (c.nwt * s);
    return b < 1 ? 1 : b;
  };
  // The LDS target keeps two or more workgroups per CU.  An unsplit launch of 160 to 256
  // workgroups (at most one round of one per CU) may use the whole LDS instead of splitting K
  // to stay under it: the down projection at M = 1 (256 workgroups, one split of 86 KB
  // instead of two of 61 KB) 31.4 -> 28.0 us, qkv at M = 5 (160 workgroups) 17.4 -> 15.5 us;
  // with fewer workgroups (o at M = 4, 5: 128) the split launch stays faster (11.7 against
  // 14.6 us), and a launch that splits anyway keeps the target (down at M = 2: 28.5 against
  // 43.1 us).
  int bpw = per_wave(splits);
  const bool whole_lds = !forced && splits == 1 && p.tiles >= 160 && p.tiles <= 256 &&
                         slice_lds_bytes(M, mv, c, c.nwt * bpw * 8) <= kSmallLdsMax;
  while (!forced && !whole_lds && bpw > 1 &&
         slice_lds_bytes(M, mv, c, c.nwt * bpw * 8) > kSliceLdsTarget)
    bpw = per_wave(++splits);
  splits = (blocks + c.nwt * bpw - 1) / (c.nwt * bpw);
  p.splits = splits;
  p.k_per_split = bpw * 8 * 128;
  p.variant = 1;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  p.reduce_launch = t(QV_TUNE_W4A16_REDUCE) == 2;
  p.ok = slice_lds_bytes(M, mv, c, c.nwt * bpw * 8) <= kSmallLdsMax &&
         (splits == 1 || p.tiles <= (int)(QV_WORKSPACE_COUNTER_BYTES / 4));
  return p;
}

}  // namespace

namespace {

// Plan of the wide kernel, configuration index cfg (kWideBase + i): about one workgroup per CU
// (K split so that tile blocks x splits is closest to the 256 CUs), every split a multiple of
// 8 groups, split partials added by the reduction launch.
GemmPlan plan_wide(int M, int N, int K, int cfg, const Tuning& t) {
  GemmPlan p{};
  const WideShape c = kWideShapes[cfg - kWideBase];
  const int groups = K / 128;
  p.waves = cfg;
  p.tiles = (N + 32 * c.nt * c.nw - 1) / (32 * c.nt * c.nw);
  int splits = (256 + p.tiles / 2) / p.tiles;
  const int max_splits = groups / 8 > 0 ? groups / 8 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  if (int e = t(QV_TUNE_W4A16_SPLITS)) splits = e;
  if (splits > groups) splits = groups;
  int gps = (groups + splits - 1) / splits;
  gps = (gps + 7) / 8 * 8;
  splits = (groups + gps - 1) / gps;
  p.splits = splits;
  p.k_per_split = gps * 128;
  p.variant = (M + 31) / 32;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  p.reduce_launch = splits > 1;
  p.ok = groups % 8 == 0;
  return p;
}

}  // namespace

GemmPlan plan_w4a16(int M, int N, int K, bool vec_ok, const Tuning& t) {
  const int groups = K / 128;
  const bool vec = vec_ok && groups % 8 == 0;
  // Default, M <= 16 with the 8-group scale/zero layout: the small-M kernels (activations as
  // the MFMA's A operand, scales applied to fp32 group sums).  Up to four tokens, and for
  // the qkv/o-sized linears up to eight, the workgroup stages its whole K range once
  // (w4a16_slice_kernel: measured on the Llama-3-70B linears at M = 1 against the chunked
  // kernel, gate_up 55.4 -> 47.1 us, down 31.1 -> 26.7 us, qkv 17.9 -> 12.7 us, o 12.4 ->
  // 9.7 us); otherwise the activations come in double-buffered chunks (w4a16_small_kernel:
  // four tiles of two waves with 4-group chunks and the zero-point MFMA for gate_up-sized and
  // long-K linears, else two tiles of four waves with 2-group chunks).
  // M > 16 with that layout: the chunked ring (activation chunks in LDS, weight ring, 8-group
  // scale/zero vectors), 8 waves of one 16-channel tile each, two groups in flight and
  // two-group chunks; with more 128-channel tiles than CUs, two tiles per wave in 7-wave
  // workgroups whose eighth wave only stages the activations (w4a16_stage_kernel).
  // Without the vector layout: the register ring for M <= 16, else the LDS-staged kernel.
  int cfg = M <= 16 ? 2 : kStagedCfg;
  if (vec) {
    if (M <= 4) {
      // Measured on the Llama-3-70B linears at M = 1..4 (interleaved timings of every
      // small-M configuration).  One token: whole-slice staging with the zero-point MFMA, two
      // tiles per workgroup of two waves each from 600 tiles (qkv, gate_up), else of four
      // (o, down).  Two to four tokens: the slice of a long K (down) outgrows the LDS from
      // M = 2, where eight one-wave tiles share it (28.3 against 35.6 us), and from M = 3 the
      // chunk-staged kernel wins (32.0 against 35.8-39.5 us); gate_up-sized linears take
      // four two-wave tiles at M = 3 (55.2 against 62.8 us) and the chunk-staged kernel at
      // M = 4 (62.0 against 71.2 us); qkv/o-sized ones four two-wave tiles at M = 2, 3
      // (qkv 13.7-14.4 against 15.2-15.4 us), and at M = 4 tiles with the zero point
      // subtracted, four of two waves (qkv) or two of four (o): retaken after the slice
      // staging went to rounds of four loads, qkv 16.97 -> 14.57 us against eight one-wave
      // tiles with the zero-point MFMA, o 11.80 -> 10.89 against four two-wave tiles.
      const bool long_k = K > 16384, wide = N / 16 >= 2048, many = N / 16 >= 600;
      const int fold_slice = kSliceBase + kFoldOffset;
      if (M == 1) cfg = fold_slice + (many ? 7 : 1);
      else if (long_k) cfg = M == 2 ? fold_slice + 2 : kSmallBase + kFoldOffset + 2;
      else if (wide) cfg = M == 2 ? fold_slice + 7 : M == 3 ? fold_slice : kSmallBase + kFoldOffset + 2;
      else if (M < 4) cfg = fold_slice + (many ? 0 : 1);
      else cfg = kSliceBase + (many ? 0 : 1);
    } else if (M <= 8 && N / 16 < 2048 && K <= 16384) {
      // qkv/o-sized, zero points subtracted: four tiles of two waves from 600 tiles, else two
      // of four (the Llama-3-70B o at M = 5, 6, 8: 12.30 -> 11.63, 12.59 -> 11.81, 13.64 ->
      // 12.70 us).
      cfg = kSliceBase + (N / 16 >= 600 ? 0 : 1);
    } else if (M <= 16) {
      // Four two-wave tiles with the zero-point MFMA for gate_up-sized and long-K linears up to
      // eight tokens; from nine, eight one-wave tiles with the zero-point MFMA (gate_up-sized:
      // 71.3 -> 68.9-69.8, 72.0 -> 68.9, 72.6 -> 70.4-70.8, 73.2 -> 70.0 us at M = 10, 12, 14,
      // 16) and four two-wave tiles with the zero points subtracted (long K, the down
      // projection: 36.5 -> 34.5, 36.7 -> 35.6, 37.6 -> 36.3, 37.8 -> 36.9 us).
      if (N / 16 >= 2048) cfg = kSmallBase + kFoldOffset + (M > 8 ? 0 : 2);
      else if (K > 16384) cfg = kSmallBase + (M > 8 ? 2 : kFoldOffset + 2);
      else cfg = kSmallBase + 5;
    } else {
      // One tile per wave, 8 waves, or 10 from 600 tiles (the Llama-3-70B qkv, 640 tiles: 64
      // workgroups x 4 splits fill the 256 CUs exactly, where 8 waves give 80 x 3; 19.6 -> 18.2,
      // 20.1 -> 19.1, 22.1 -> 21.3, 23.0 -> 22.6, 26.6 -> 25.9 us at M = 17, 28, 33, 48, 64).
      cfg = N / 16 >= 600 ? kChunkBase + 9 : kChunkBase + 4;
      if ((N + 127) / 128 > 256) {
        // Two tiles per wave in 7 compute waves plus a staging wave, 224 channels per
        // workgroup (the Llama-3-70B gate_up in 256 workgroups): two-group weight ring and
        // 4-group chunks up to 48 tokens, 4-group ring and 2-group chunks above (one staging
        // wave holds a whole chunk).  Measured on that linear against the kernels it
        // replaced (the wide kernel up to 32 tokens, the 7-wave chunk kernel to 48, the
        // 8-wave one above): 66-67 against 70-72 us at 17-32 tokens, 72-75 against 76-78 at
        // 33-48, 87-88 against 88-90 at 49-64.
        cfg = kStageBase + (M > 48 ? 2 : 1);
      }
    }
  }
  if (int e = t(QV_TUNE_W4A16_CFG)) {
    if ((e >= 1 && e < kNumRing) || e == kStagedCfg) cfg = e;
    else if (vec && e >= kChunkBase && e < kChunkBase + kNumChunkShapes) cfg = e;
    else if (vec && e >= kWideBase && e < kWideBase + kNumWideShapes) cfg = e;
    else if (vec && e >= kStageBase && e < kStageBase + kNumStageShapes &&
             stage_fits(M, kStageShapes[e - kStageBase].cg))
      cfg = e;
    else if (vec && M <= 16 && ((e >= kSmallBase && e < kSmallBase + kNumSmallShapes) ||
                                (e >= kSmallBase + kFoldOffset &&
                                 e < kSmallBase + kFoldOffset + kNumSmallShapes)))
      cfg = e;
    else if (vec && M <= 16 && ((e >= kSliceBase && e < kSliceBase + kNumSliceShapes) ||
                                (e >= kSliceBase + kFoldOffset &&
                                 e < kSliceBase + kFoldOffset + kNumSliceShapes)))
      cfg = e;
  }
  if (cfg >= kWideBase && cfg < kStageBase) return plan_wide(M, N, K, cfg, t);
  if (cfg >= kSliceBase && cfg < kWideBase) {
    const GemmPlan ps = plan_slice(M, N, K, cfg, t);
    if (ps.ok) return ps;
    cfg = kSmallBase + (N / 16 >= 2048 ? 0 : M <= 4 ? 1 : 5);  // the slice does not fit in LDS
  }
  if (cfg >= kSmallBase && cfg < kSliceBase) return plan_small(M, N, K, cfg, t);

  GemmPlan p{};
  p.waves = cfg;
  int splits;
  int gps_max = groups;
  int gps_align = 1;
  if (cfg == kStagedCfg) {
    const int rows = kNW * kNT * 16;
    p.tiles = (N + rows - 1) / rows;
    const int target = 512;
    splits = (target + p.tiles - 1) / p.tiles;
    const int max_splits = groups / (2 * kCG) > 0 ? groups / (2 * kCG) : 1;
    if (splits > max_splits) splits = max_splits;
  } else if (cfg < kChunkBase) {
    const RingCfg c = kRing[cfg];
    const int rows = c.nt * c.nw * 16;
    p.tiles = (N + rows - 1) / rows;
    // About 16 waves per CU in total and at least P groups per split; the staged slice
    // (M rows) must fit in the LDS of one CU.
    const int target_wgs = 4096 / c.nw;
    splits = (target_wgs + p.tiles - 1) / p.tiles;
    const int max_splits = groups / c.p > 0 ? groups / c.p : 1;
    if (splits > max_splits) splits = max_splits;
    gps_max = (int)(kRingLdsMax / ((size_t)M * 16 * sizeof(u32x4)));
    if (groups % 8 == 0) gps_align = 8;
  } else {
    const int rows = cfg >= kStageBase
                         ? kStageShapes[cfg - kStageBase].nt * kStageShapes[cfg - kStageBase].nw * 16
                         : kChunkShapes[cfg - kChunkBase].nt * kChunkShapes[cfg - kChunkBase].nw * 16;
    p.tiles = (N + rows - 1) / rows;
    // About one workgroup per CU: split K so that tiles x splits is closest to the 256 CUs.
    // Measured on the Llama-3-70B shapes at M = 1, 5 and 48, fewer and longer workgroups
    // beat more and shorter ones, which pay the prologue and the split-K exchange more often.
    splits = (256 + p.tiles / 2) / p.tiles;
    const int max_splits = groups / 8 > 0 ? groups / 8 : 1;
    if (splits > max_splits) splits = max_splits;
    gps_align = 8;
  }
  if (splits < 1) splits = 1;
  if (int e = t(QV_TUNE_W4A16_SPLITS)) splits = e;
  if (splits > groups) splits = groups;
  int gps = (groups + splits - 1) / splits;
  if (gps_align > 1) {
    gps = (gps + gps_align - 1) / gps_align * gps_align;
    if (gps_max >= gps_align) gps_max = gps_max / gps_align * gps_align;
  }
  if (gps > gps_max) gps = gps_max;
  if (gps < 1) gps = 1;
  splits = (groups + gps - 1) / gps;
  p.splits = splits;
  p.k_per_split = gps * 128;
  p.variant = (M + 15) / 16;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  // Above 16 tokens the split-K partials go through a second launch: at M = 48 the arrival
  // round trips of the in-kernel finish (write-through stores, their completion, the counter,
  // the last workgroup's coherent loads) cost 7-8 us per launch, the second launch 3-4 us
  // (Llama-3-70B qkv 27.7 -> 24.2 us, o 23.7 -> 20.1, down 51.2 -> 47.2); at M <= 16 the two
  // are level, and one launch is kept.
  const int red = t(QV_TUNE_W4A16_REDUCE);
  p.reduce_launch = cfg >= kStageBase || (cfg >= kChunkBase && (red == 2 || (red == 0 && M > 16)));
  // One arrival counter per tile block in the workspace's counter region: a split plan with
  // more tile blocks than counters is refused (only past about two million channels).
  p.ok = splits == 1 || p.tiles <= (int)(QV_WORKSPACE_COUNTER_BYTES / 4);
  return p;
}

// The split-K finish as a launch of its own: thread i adds outputs 4i .. 4i + 3 of the M x N
// result (row-major) over the splits in split order, four splits' loads in flight before any
// of them is added, multiplies by the row's scale if there is one, and stores them as fp16.
// The sum starts from +0 and adds split 0 first, as the in-kernel finishes do, so both
// finishes give the same bits.
__global__ __launch_bounds__(256) void reduce_splits_kernel(const f32x4* __restrict__ part,
                                                            int splits, int n4, int n4_row,
                                                            const float* __restrict__ row_scale,
                                                            uint16_t* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += 4) {
    f32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = part[(size_t)min(s0 + j, splits - 1) * n4 + i];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (s0 + j < splits) t += v[j];
  }
  uint32_t lo, hi;
  if (row_scale) {
    const float sc = row_scale[i / n4_row];
    lo = (uint32_t)f16_of_product(t[0], sc) | ((uint32_t)f16_of_product(t[1], sc) << 16);
    hi = (uint32_t)f16_of_product(t[2], sc) | ((uint32_t)f16_of_product(t[3], sc) << 16);
  } else {
    lo = __builtin_bit_cast(uint32_t, f16x2{(_Float16)t[0], (_Float16)t[1]});
    hi = __builtin_bit_cast(uint32_t, f16x2{(_Float16)t[2], (_Float16)t[3]});
  }
  *reinterpret_cast<u32x2*>(y + (size_t)i * 4) = u32x2{lo, hi};
}

hipError_t launch_reduce_splits(const float* part, int splits, int M, int N,
                                const float* row_scale, uint16_t* y, hipStream_t stream) {
  const long long n4 = (long long)M * N / 4;
  if (splits < 1 || N % 4 != 0 || n4 < 1 || n4 > INT32_MAX) return hipErrorInvalidValue;
  const int blocks = (int)((n4 + 255) / 256);
  reduce_splits_kernel<<<blocks, 256, 0, stream>>>(reinterpret_cast<const f32x4*>(part), splits,
                                                   (int)n4, N / 4, row_scale, y);
  return hipGetLastError();
}

hipError_t launch_w4a16(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream) {
  if (p.waves >= kStageBase)
    return launch_stage(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
  if (p.waves >= kWideBase)
    return launch_wide(p, x, M, K, qw, scales, zeros, N, y, partials, stream);
  if (p.waves >= kSliceBase)
    return launch_slice(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  if (p.waves >= kSmallBase)
    return launch_small(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
  switch (p.variant) {
    case 1: return launch_mt<1>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 2: return launch_mt<2>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 3: return launch_mt<3>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 4: return launch_mt<4>(p, x, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qv
