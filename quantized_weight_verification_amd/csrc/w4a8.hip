// W4A8 linear: 4-bit weights (group 128, fp16 scale and 0..15 zero point per group, eight
// codes per 32-bit word) against per-token int8 activations, on the int8 matrix cores
// (Speculative Decoding Meets Quantization, review page: the W4A8 target beside W4A16).
//
//   acc_g[m][n] = sum_{k in group g} x_q[m][k] * (q[n][k] - z[n][g])     (exact int32)
//   y[m][n]     = fp16( x_scale[m] * sum_g s[n][g] * acc_g[m][n] )        (fp32 sum over g)
//
// Up to 16 tokens the zero point is applied after the product: the MFMA multiplies the raw
// codes (0..15 as int8) and each group's result is corrected by z * sum_{k in g} x_q[m][k], an
// integer the staging pass computes once per (token, group).  Above 16 tokens the correction
// would cost four integer operations per output and token tile, so the chunked kernel
// subtracts each lane's zero point from its own codes before the MFMA instead (two operations
// per word of four codes); both give the same exact int32 group sums.  A code word is unpacked with two masks and
// a shift into the bytes of k = 0,2,4,6 and k = 1,3,5,7; the staged activations carry the
// same permutation inside every 8 bytes, so the int8 products pair up unchanged.
//
// Work split: a workgroup owns NT tiles of 16 channels and a K-slice of whole groups (split
// across workgroups when needed); NWT waves per tile divide that slice.  The slice's x_q rows
// (permuted and XOR-swizzled by 16-byte column), their per-group sums, and the tiles' scales
// and zero points are staged in LDS once; then each wave streams its weight rows through a
// P-group register ring (one 16-byte load per lane per group, two v_mfma_i32_16x16x64_i8 per
// 16-token tile), folding each group into fp32 accumulators.  Waves are summed through LDS in
// wave order; with split-K each slice stores fp32 partials (agent-scope coherent) and the
// last workgroup of the tile group adds them in split order and applies x_scale.  Batches of
// more than 16 tokens use w4a8_chunk_kernel (below), which streams K in double-buffered
// activation chunks instead of splitting it.
#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kGroup = QV_W4A16_GROUP;  // 128
constexpr int kP = 8;                   // groups in flight per lane
constexpr size_t kLdsMax = 64 * 1024;   // staged slice budget per workgroup

__device__ __forceinline__ int byte_sum(uint32_t d) {
  return (int)(int8_t)(d & 0xFFu) + (int)(int8_t)((d >> 8) & 0xFFu) +
         (int)(int8_t)((d >> 16) & 0xFFu) + (int)(int8_t)(d >> 24);
}

// Bytes b0..b15 of a 16-byte vector -> b0 b2 b4 b6 | b1 b3 b5 b7 | b8 b10 b12 b14 |
// b9 b11 b13 b15 (the order of the unpacked codes).
__device__ __forceinline__ u32x4 permute16(u32x4 t) {
  return u32x4{__builtin_amdgcn_perm(t[1], t[0], 0x06040200u),
               __builtin_amdgcn_perm(t[1], t[0], 0x07050301u),
               __builtin_amdgcn_perm(t[3], t[2], 0x06040200u),
               __builtin_amdgcn_perm(t[3], t[2], 0x07050301u)};
}

struct Lds {
  // offsets in bytes into the dynamic LDS block
  size_t xs, xsum, scl, zer, total;
};

__host__ __device__ inline size_t align16(size_t b) { return (b + 15) & ~(size_t)15; }

// Staged slice of gs groups: x_q rows [M][vpr] 16-byte vectors, their group sums [M][gs]
// int32, the channels' scales [gs][nt*16] fp32 and zero points [gs][nt*16] bytes; each part
// 16-byte aligned.
__host__ __device__ inline Lds lds_layout(int M, int gs, int nt) {
  Lds l;
  const int vpr = ((gs * 8 + 15) / 16) * 16;  // 16-byte vectors per staged row
  l.xs = 0;
  l.xsum = (size_t)M * vpr * 16;
  l.scl = align16(l.xsum + (size_t)M * gs * 4);
  l.zer = align16(l.scl + (size_t)gs * nt * 16 * 4);
  l.total = align16(l.zer + (size_t)gs * nt * 16);
  return l;
}

template <int MT, int NT, int NWT>
__global__ __launch_bounds__(NT * NWT * 64) void w4a8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int M, int K,
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int N, uint16_t* __restrict__ y,
    unsigned* __restrict__ counters, float* __restrict__ part, int splits, int gps) {
  constexpr int NW = NT * NWT;
  constexpr int NTH = NW * 64;
  extern __shared__ __align__(16) unsigned char lds[];
  const int grp = blockIdx.x, split = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;
  const int it = wave / NWT, wt = wave % NWT;
  const int nbase = grp * NT * 16;
  const int n0 = nbase + it * 16;
  const int G = K / kGroup;
  const int gb = split * gps;
  const int ge = min(gb + gps, G);
  const int gs = ge - gb;  // groups in this slice
  const int g0 = gb + (gs * wt) / NWT, g1 = gb + (gs * (wt + 1)) / NWT;
  const Lds L = lds_layout(M, gps, NT);
  const int vpr = ((gps * 8 + 15) / 16) * 16;
  u32x4* xs = reinterpret_cast<u32x4*>(lds + L.xs);
  int* xsum = reinterpret_cast<int*>(lds + L.xsum);       // [M][gps]
  float* scl = reinterpret_cast<float*>(lds + L.scl);     // [gps][NT*16]
  uint8_t* zer = lds + L.zer;                             // [gps][NT*16]

  // The weight ring: lane (r, kg) holds dwords 4kg .. 4kg+3 of group g of channel n0 + r.
  // Every ring load is issued unconditionally, its group clamped to the wave's last one (a
  // wave without groups reads a valid group it never uses): a load behind a `group < end`
  // test made the compiled loop wait for all loads in flight at every group, so only one
  // group per lane was ever in flight.
  const uint32_t* wp = qw + (size_t)(n0 + r) * (K / 8) + kg * 4;
  const int gclamp = min(max(g1 - 1, g0), G - 1);
  u32x4 wq[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p)
    wq[p] = *reinterpret_cast<const u32x4*>(wp + (size_t)min(g0 + p, gclamp) * 16);

  // Stage the slice: x_q rows (permuted, swizzled) with per-(token, group) sums, eight
  // 16-byte vectors per group.  The eight vectors of one group sit in eight consecutive
  // lanes, which add their byte sums by shuffles.
  const int vrow = gs * 8;
  const int nvec = M * vrow;
  for (int e0 = threadIdx.x; e0 < ((nvec + 7) & ~7); e0 += 4 * NTH) {
    u32x4 d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = min(e0 + j * NTH, nvec - 1);
      const int m = e / vrow, v = e - m * vrow;
      d[j] = *reinterpret_cast<const u32x4*>(xq + (size_t)m * K + (size_t)gb * kGroup + v * 16);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * NTH;
      int s = byte_sum(d[j][0]) + byte_sum(d[j][1]) + byte_sum(d[j][2]) + byte_sum(d[j][3]);
      s += __shfl_xor(s, 1, kWave);
      s += __shfl_xor(s, 2, kWave);
      s += __shfl_xor(s, 4, kWave);
      if (e < nvec) {
        const int m = e / vrow, v = e - m * vrow;
        xs[m * vpr + (v ^ (m & 15))] = permute16(d[j]);
        if ((v & 7) == 0) xsum[m * gps + (v >> 3)] = s;
      }
    }
  }
  // Scales (as fp32) and zero points of the workgroup's channels for the slice's groups.
  for (int e = threadIdx.x; e < NT * 16 * gs; e += NTH) {
    const int c = e / gs, g = e - c * gs;
    const size_t src = (size_t)(nbase + c) * G + gb + g;
    scl[g * NT * 16 + c] = (float)__builtin_bit_cast(_Float16, scales[src]);
    zer[g * NT * 16 + c] = zeros[src];
  }
  __syncthreads();

  int brow[MT], bkey[MT], tok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
    tok[mt] = m;
    brow[mt] = m * vpr;
    bkey[mt] = m & 15;
  }
  f32x4 facc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) facc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int cbase = it * 16 + kg * 4;  // this lane's four accumulator channels in the group
  // One group from ring slot p: two MFMAs per token tile on the raw codes, then the zero-point
  // correction and one FMA with the scale per output.
  auto group = [&](int p, int gl) {
    const u32x4 wv = wq[p];
    i32x4 ai[MT];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d0 = wv[2 * h], d1 = wv[2 * h + 1];
      const i32x4 A = {(int)(d0 & 0x0F0F0F0Fu), (int)((d0 >> 4) & 0x0F0F0F0Fu),
                       (int)(d1 & 0x0F0F0F0Fu), (int)((d1 >> 4) & 0x0F0F0F0Fu)};
      const int v = gl * 8 + kg * 2 + h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x4 B = __builtin_bit_cast(i32x4, xs[brow[mt] + (v ^ bkey[mt])]);
        ai[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, h ? ai[mt] : i32x4{0, 0, 0, 0}, 0, 0, 0);
      }
    }
    return [&, gl, ai]() mutable {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(&scl[gl * NT * 16 + cbase]);
      const uint32_t zz = *reinterpret_cast<const uint32_t*>(&zer[gl * NT * 16 + cbase]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int xsg = xsum[tok[mt] * gps + gl];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int z = (int)((zz >> (8 * v)) & 0xFFu);
          facc[mt][v] += sc[v] * (float)(ai[mt][v] - z * xsg);
        }
      }
    };
  };
  // Whole batches of kP groups while more groups follow them: every refill is issued
  // unconditionally (groups past the end clamped to the wave's last one), so the compiled loop
  // waits for one load at a time.  (A refill behind a `group < end` test, vector or scalar,
  // made it wait for all loads in flight at every group or every batch: 20-45 % slower.)  The
  // last 1..kP groups, already in the ring, follow without refills, each waiting only for its
  // own slot.
  int g = g0;
  for (; g + kP < g1; g += kP) {
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      auto finish = group(p, g + p - gb);
      wq[p] = *reinterpret_cast<const u32x4*>(wp + (size_t)min(g + p + kP, gclamp) * 16);
      __builtin_amdgcn_sched_barrier(0);
      finish();
    }
  }
#pragma unroll
  for (int p = 0; p < kP; ++p)
    if (g + p < g1) group(p, g + p - gb)();

  // Sum the waves of each tile through LDS (in wave order), reusing the staging space.
  __syncthreads();
  float(*red)[MT][16][16] = reinterpret_cast<float(*)[MT][16][16]>(lds);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4*>(&red[wave][mt][r][kg * 4]) = facc[mt];
  __syncthreads();

  constexpr int OUT = NT * MT * 256;
  constexpr int EPT = (OUT + NTH - 1) / NTH;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NTH;
    const int ti = t / (MT * 256), u = t % (MT * 256);
    const int mt = u >> 8, j = (u >> 4) & 15, i = u & 15;
    const int m = mt * 16 + j;
    if (t >= OUT || m >= M) continue;
    float sum = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWT; ++wv) sum += red[ti * NWT + wv][mt][j][i];
    const int n = nbase + ti * 16 + i;
    if (splits == 1)
      y[(size_t)m * N + n] = f16_of_product(sum, sx[m]);
    else
      st_coherent(&part[((size_t)split * M + m) * N + n], sum);
  }
  if (splits == 1) return;
  if (!arrive_last(&counters[grp], (unsigned)splits)) return;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NTH;
    const int ti = t / (MT * 256), u = t % (MT * 256);
    const int mt = u >> 8, j = (u >> 4) & 15, i = u & 15;
    const int m = mt * 16 + j;
    if (t >= OUT || m >= M) continue;
    const int n = nbase + ti * 16 + i;
    // Eight splits' loads in flight before any is added; added in split order.
    float sum = 0.f;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = ld_coherent(&part[((size_t)min(sp0 + q, splits - 1) * M + m) * N + n]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (sp0 + q < splits) sum += v[q];
    }
    y[(size_t)m * N + n] = f16_of_product(sum, sx[m]);
  }
}

// Chunked variant for tree-sized batches (M > 16), where a slice of K staged whole leaves
// room for only a few groups and split-K partials would outweigh the weights.  Each of the
// NT waves owns one 16-channel tile and streams it over the workgroup's whole K range; the
// activations pass through LDS in chunks of CG groups, double-buffered: the loads of chunk
// c + 1 are issued before chunk c is multiplied and stored to the other buffer after it.
// The weight ring holds CG groups per lane (slot i serves group i of every chunk).  K is
// split across workgroups only to give the launch enough workgroups.
template <int MT, int NT, int CG>
__global__ __launch_bounds__(NT * 64) void w4a8_chunk_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int M, int K,
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int N, uint16_t* __restrict__ y,
    unsigned* __restrict__ counters, float* __restrict__ part, int splits, int gps,
    int reduce_launch) {
  constexpr int NTH = NT * 64;
  constexpr int VPC = CG * 8;                     // 16-byte x vectors per row per chunk
  constexpr int CVPR = ((VPC + 15) / 16) * 16;    // ... per staged row (swizzle period)
  constexpr int XV = (64 * VPC + NTH - 1) / NTH;  // staging vectors per thread (M <= 64)
  constexpr int SV = (NT * 16 * CG + NTH - 1) / NTH;
  extern __shared__ __align__(16) unsigned char lds[];
  const int grp = blockIdx.x, split = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, kg = lane >> 4;
  const int nbase = grp * NT * 16;
  const int n0 = nbase + wave * 16;
  const int G = K / kGroup;
  const int gb = split * gps;
  const int ge = min(gb + gps, G);
  const int nch = (ge - gb + CG - 1) / CG;
  // One buffer: x rows [M][CVPR] vectors, scales [CG][NT*16] fp32, zero points [CG][NT*16]
  // bytes.
  const size_t xs_b = (size_t)M * CVPR * 16;
  const size_t scl_o = align16(xs_b);
  const size_t zer_o = align16(scl_o + (size_t)CG * NT * 16 * 4);
  const size_t buf_b = align16(zer_o + (size_t)CG * NT * 16);

  const uint32_t* wp = qw + (size_t)(n0 + r) * (K / 8) + kg * 4;
  u32x4 wq[CG];
#pragma unroll
  for (int i = 0; i < CG; ++i)
    if (gb + i < ge) wq[i] = *reinterpret_cast<const u32x4*>(wp + (size_t)(gb + i) * 16);

  // Loads of chunk c (clamped, unconditional) and their store into buffer b.
  u32x4 xv[XV];
  uint16_t sv[SV];
  uint8_t zv[SV];
  auto load_chunk = [&](int c) {
    const int cg0 = gb + c * CG;
    const int gl = min(CG, ge - cg0);
    const int nv = M * gl * 8;
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = min((int)threadIdx.x + j * NTH, nv - 1);
      const int m = e / (gl * 8), v = e - m * (gl * 8);
      xv[j] = *reinterpret_cast<const u32x4*>(xq + (size_t)m * K + (size_t)cg0 * kGroup + v * 16);
    }
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      const int e = min((int)threadIdx.x + j * NTH, NT * 16 * gl - 1);
      const int ch = e / gl, g = e - ch * gl;
      const size_t src = (size_t)(nbase + ch) * G + cg0 + g;
      sv[j] = scales[src];
      zv[j] = zeros[src];
    }
  };
  auto store_chunk = [&](int c, int b) {
    unsigned char* base = lds + (size_t)b * buf_b;
    u32x4* xs = reinterpret_cast<u32x4*>(base);
    float* scl = reinterpret_cast<float*>(base + scl_o);
    uint8_t* zer = base + zer_o;
    const int cg0 = gb + c * CG;
    const int gl = min(CG, ge - cg0);
    const int nv = M * gl * 8;
    // Threads past the chunk's last vector (or scale) store the copy of it that their clamped
    // load fetched, to its own place: identical values, and no branch around the stores.  (A
    // store under an `e < nv` test let the compiler sink its load into that branch, next to
    // the store, where the wait for it also drained the weight ring at every chunk.)
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      const int e = min((int)threadIdx.x + j * NTH, nv - 1);
      const int m = e / (gl * 8), v = e - m * (gl * 8);
      xs[m * CVPR + (v ^ (m & 15))] = permute16(xv[j]);
    }
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      const int e = min((int)threadIdx.x + j * NTH, NT * 16 * gl - 1);
      const int ch = e / gl, g = e - ch * gl;
      scl[g * NT * 16 + ch] = (float)__builtin_bit_cast(_Float16, sv[j]);
      zer[g * NT * 16 + ch] = zv[j];
    }
  };

  int brow[MT], bkey[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
    brow[mt] = m * CVPR;
    bkey[mt] = m & 15;
  }
  f32x4 facc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) facc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int cbase = wave * 16 + kg * 4;

  // Group i of chunk c (ring slot i): the MFMAs into ai, then (after the slot's refill is
  // issued) the fp32 accumulation.
  i32x4 ai[MT];
  auto mfmas = [&](int c, int i) {
    const unsigned char* base = lds + (size_t)(c & 1) * buf_b;
    const u32x4* xs = reinterpret_cast<const u32x4*>(base);
    const uint8_t* zer = base + zer_o;
    const u32x4 wv = wq[i];
    // The zero point of this lane's weight row (channel n0 + r) leaves the codes before the
    // MFMA: each byte becomes code - zero as int8 (exact, -15..15), so the MFMA sums x_q *
    // (code - zero) directly.  A byte c (0..15) with its top bit set is c + 128; adding the
    // two's complement of zero * 0x01010101 subtracts the zero from every byte without a
    // borrow between bytes (c + 128 - zero >= 113), and clearing the top bit again by XOR
    // leaves c - zero in two's complement.
    const uint32_t zown = zer[i * NT * 16 + wave * 16 + r];
    const uint32_t nzz = 0u - zown * 0x01010101u;
    auto minus_zero = [&](uint32_t u) { return (int)(((u ^ 0x80808080u) + nzz) ^ 0x80808080u); };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d0 = wv[2 * h], d1 = wv[2 * h + 1];
      const i32x4 A = {minus_zero(d0 & 0x0F0F0F0Fu), minus_zero((d0 >> 4) & 0x0F0F0F0Fu),
                       minus_zero(d1 & 0x0F0F0F0Fu), minus_zero((d1 >> 4) & 0x0F0F0F0Fu)};
      const int v = i * 8 + kg * 2 + h;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x4 B = __builtin_bit_cast(i32x4, xs[brow[mt] + (v ^ bkey[mt])]);
        ai[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, h ? ai[mt] : i32x4{0, 0, 0, 0}, 0, 0, 0);
      }
    }
  };
  auto accumulate = [&](int c, int i) {
    const float* scl = reinterpret_cast<const float*>(lds + (size_t)(c & 1) * buf_b + scl_o);
    const f32x4 sc = *reinterpret_cast<const f32x4*>(&scl[i * NT * 16 + cbase]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v) facc[mt][v] += sc[v] * (float)ai[mt][v];
  };

  // Every chunk but the last has all CG groups and a successor: its chunk loads and weight
  // refills are issued unconditionally (refills past the end clamped to the last group), so
  // the compiled loop waits for one load at a time (a load behind a `group < end` test made it
  // wait for all loads in flight at every group; measured at 17-48 tokens: gate_up 86.7 ->
  // 77.3 us at M = 17, 90.5 -> 86.6 at M = 48, qkv 25.3 -> 24.4 at M = 48).  The last chunk's
  // groups, already in the ring, follow without refills.  (With four token tiles this form
  // spilled until the chunk stores lost their branches; now it fits in 128 VGPRs and took the
  // Llama-3-70B linears at M = 64 from 95 to 80 us (gate_up), 55 to 47 (down), 28 to 25 (qkv).)
  load_chunk(0);
  store_chunk(0, 0);
  __syncthreads();
  for (int c = 0; c + 1 < nch; ++c) {
    load_chunk(c + 1);
#pragma unroll
    for (int i = 0; i < CG; ++i) {
      const int gg = gb + c * CG + i;
      mfmas(c, i);
      wq[i] = *reinterpret_cast<const u32x4*>(wp + (size_t)min(gg + CG, ge - 1) * 16);
      __builtin_amdgcn_sched_barrier(0);
      accumulate(c, i);
    }
    store_chunk(c + 1, (c + 1) & 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < CG; ++i) {
    if (gb + (nch - 1) * CG + i < ge) {
      mfmas(nch - 1, i);
      accumulate(nch - 1, i);
    }
  }

  // Each wave owns its tile: lane (r, kg) holds channels n0 + 4kg .. +3 of token mt*16 + r.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + r;
    if (m >= M) continue;
    const int n = n0 + kg * 4;
    if (splits == 1) {
      const float t = sx[m];
      uint32_t lo = (uint32_t)f16_of_product(facc[mt][0], t) |
                    ((uint32_t)f16_of_product(facc[mt][1], t) << 16);
      uint32_t hi = (uint32_t)f16_of_product(facc[mt][2], t) |
                    ((uint32_t)f16_of_product(facc[mt][3], t) << 16);
      *reinterpret_cast<u32x2*>(&y[(size_t)m * N + n]) = u32x2{lo, hi};
    } else if (reduce_launch) {  // a second launch adds the splits: plain stores
      *reinterpret_cast<f32x4*>(&part[((size_t)split * M + m) * N + n]) = facc[mt];
    } else {
      st_coherent_f4(&part[((size_t)split * M + m) * N + n], facc[mt]);
    }
  }
  if (splits == 1 || reduce_launch) return;
  if (!arrive_last(&counters[grp], (unsigned)splits)) return;
  // The last slice adds the partials of the workgroup's NT * 16 channels in split order.
  for (int t = threadIdx.x; t < M * NT * 4; t += NTH) {
    const int m = t / (NT * 4), n = nbase + (t - m * (NT * 4)) * 4;
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < splits; ++sp) sum += ld_coherent_f4(&part[((size_t)sp * M + m) * N + n]);
    const float sc = sx[m];
    uint32_t lo = (uint32_t)f16_of_product(sum[0], sc) |
                  ((uint32_t)f16_of_product(sum[1], sc) << 16);
    uint32_t hi = (uint32_t)f16_of_product(sum[2], sc) |
                  ((uint32_t)f16_of_product(sum[3], sc) << 16);
    *reinterpret_cast<u32x2*>(&y[(size_t)m * N + n]) = u32x2{lo, hi};
  }
}

size_t chunk_lds_bytes(int M, int nt, int cg) {
  const int cvpr = ((cg * 8 + 15) / 16) * 16;
  size_t b = (size_t)M * cvpr * 16;
  b = align16(b);
  b = align16(b + (size_t)cg * nt * 16 * 4);
  b = align16(b + (size_t)cg * nt * 16);
  return 2 * b;
}

template <int MT, int NT, int NWT>
hipError_t launch_t(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                    const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                    uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
  const int gps = p.k_per_split / kGroup;
  const Lds L = lds_layout(M, gps, NT);
  const size_t red = (size_t)NT * NWT * MT * 256 * sizeof(float);
  const size_t lds = L.total > red ? L.total : red;
  auto kern = w4a8_kernel<MT, NT, NWT>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles / NT, p.splits);
  kern<<<grid, NT * NWT * 64, lds, stream>>>(xq, sx, M, K, qw, scales, zeros, N, y, counters,
                                             static_cast<float*>(partials), p.splits, gps);
  return hipGetLastError();
}

template <int MT, int NT, int CG>
hipError_t launch_chunk(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                        const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                        uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
  const size_t lds = chunk_lds_bytes(M, NT, CG);
  auto kern = w4a8_chunk_kernel<MT, NT, CG>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles / NT, p.splits);
  const bool red = p.splits > 1 && p.reduce_launch;
  kern<<<grid, NT * 64, lds, stream>>>(xq, sx, M, K, qw, scales, zeros, N, y, counters,
                                       static_cast<float*>(partials), p.splits,
                                       p.k_per_split / kGroup, red ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !red) return e;
  return launch_reduce_splits(static_cast<const float*>(partials), p.splits, M, N, sx, y, stream);
}

template <int MT>
hipError_t launch_m(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                    const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                    uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
#define QV_W4A8_CASE(NT_, NWT_)                                                               \
  if (p.nt == NT_ && p.waves == NWT_)                                                        \
    return launch_t<MT, NT_, NWT_>(p, xq, sx, M, K, qw, scales, zeros, N, y, counters,        \
                                   partials, stream);
  QV_W4A8_CASE(1, 4)
  QV_W4A8_CASE(1, 8)
  QV_W4A8_CASE(1, 16)
  QV_W4A8_CASE(2, 4)
  QV_W4A8_CASE(4, 2)
  QV_W4A8_CASE(4, 4)
#undef QV_W4A8_CASE
  return hipErrorInvalidValue;
}

}  // namespace

// Work split: 16-channel tiles, NT per workgroup (4 from M = 2 on, sharing one staged slice,
// with 2 waves each; 1 at M = 1, with 4, 8 or 16 waves); K is split across workgroups when
// the launch would have fewer than about 2048 waves or the staged slice would exceed the LDS
// budget.
GemmPlan plan_w4a8(int M, int N, int K, const Tuning& t) {
  GemmPlan p{};
  p.tiles = N / 16;
  const int G = K / kGroup;
  // Tree-sized batches (M > 16): the chunked kernel, 16 tiles (one wave each) per workgroup
  // (8 if 16 do not divide the tiles), chunks of 4 groups; K split only as far as the
  // workgroups still fit on the 256 CUs in one round (one such workgroup per CU).  Measured on
  // the Llama-3-70B linears at M = 48: gate_up 107 us and down 56 us, against 123 / 74 us with
  // 8 tiles and 187 / 103 us with the staged-slice kernel; rounding the split count down
  // rather than up (qkv 7 -> 6 splits, 280 -> 240 workgroups; gate_up 2 -> 1) took qkv from
  // 37.7 to 30.0 us and gate_up from 112.9 to 105.6 us.  Chunks of 8 groups (a ring twice as
  // deep) for gate_up-sized linears up to three token tiles: 66.6-76.1 against 71.6-81.0 us
  // at 17-48 tokens; the narrower linears were slower with them, and four token tiles spill.
  // (For these plans `waves` holds the chunk size CG.)
  if (M > 16 && p.tiles % 8 == 0 && !t(QV_TUNE_W4A8_STAGED)) {
    p.waves = p.tiles >= 2048 && M <= 48 ? 8 : 4;
    if (int e = t(QV_TUNE_W4A8_CG)) p.waves = e >= 8 ? 8 : 4;
    p.nt = p.tiles % 16 == 0 ? 16 : 8;
    // Short linears of at most 512 tiles (the Llama-3-70B o: 64 workgroups x 4 splits instead
    // of 32 x 8, half the split partials) take 8: 16.3 -> 15.4, 16.4 -> 15.7, 19.1 -> 18.5,
    // 19.9 -> 18.7, 22.3 -> 21.5 us at M = 17, 24, 33, 48, 64 (qkv, 640 tiles, level; the
    // 224-group down slower).
    if (p.tiles <= 512 && G <= 64) p.nt = 8;
    // 14 where 16 would leave CUs idle and 14 fill them in one round, up to three token tiles
    // (the Llama-3-70B gate_up, 3584 tiles, in 256 workgroups instead of 224: 69.6 -> 67.5,
    // 67.4 -> 65.2, 73.8 -> 71.7, 75.7 -> 73.3 us at M = 17, 24, 33, 48; at M = 64, with
    // 4-group chunks, 80.5 -> 83.4, so 16 stay there).
    if (M <= 48 && p.nt == 16 && p.tiles / 16 < 256 && p.tiles % 14 == 0 && p.tiles / 14 <= 256)
      p.nt = 14;
    // 10 where 16 leave CUs idle and 10 fill more of them in one round (the Llama-3-70B qkv,
    // 640 tiles: 64 workgroups x 4 splits instead of 40 x 6; 19.20 -> 18.48, 19.73 -> 18.78,
    // 20.50 -> 19.31, 23.21 -> 21.47, 25.84 -> 24.48 us at M = 17, 24, 32, 48, 64).
    if (p.nt == 16 && p.tiles % 10 == 0) {
      const int ms = G / (2 * p.waves) > 0 ? G / (2 * p.waves) : 1;
      auto fill = [&](int nt) {
        const int w = p.tiles / nt;
        const int s = 256 / w < ms ? 256 / w : ms;
        return w * (s > 1 ? s : 1);
      };
      if (fill(10) > fill(16) && fill(10) <= 256) p.nt = 10;
    }
    if (int e = t(QV_TUNE_W4A8_NT))
      p.nt = e == 10 && p.tiles % 10 == 0   ? 10
             : e == 14 && p.tiles % 14 == 0 ? 14
             : e >= 16 && p.tiles % 16 == 0 ? 16
                                            : 8;
    if (p.nt > 8 && chunk_lds_bytes(M, p.nt, p.waves) > 160 * 1024) p.nt = 8;
    const int wgs = p.tiles / p.nt;
    int splits = 256 / wgs;
    const int max_splits = G / (2 * p.waves) > 0 ? G / (2 * p.waves) : 1;  // >= 2 chunks each
    if (splits > max_splits) splits = max_splits;
    if (int e = t(QV_TUNE_W4A8_SPLITS)) splits = e;
    if (splits < 1) splits = 1;
    if (splits > G) splits = G;
    const int gps = (G + splits - 1) / splits;
    p.splits = (G + gps - 1) / gps;
    p.k_per_split = gps * kGroup;
    p.variant = 16 + (M + 15) / 16;
    p.partial_bytes = p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
    // The split sums go through a second launch unless overridden (as for W4A16 above 16
    // tokens: the arrival round trips of the in-kernel finish cost more than a launch).
    p.reduce_launch = t(QV_TUNE_W4A8_REDUCE) != 1;
    p.ok = chunk_lds_bytes(M, p.nt, p.waves) <= 156 * 1024 &&
           (p.splits == 1 || wgs <= (int)(QV_WORKSPACE_COUNTER_BYTES / 4));
    return p;
  }
  // One token: every tile streams alone, 4 waves per tile from 640 tiles, 8 from 384 (4 when
  // K holds fewer than 128 groups, so that each wave streams at least 16), else 16 (measured
  // on the Llama-3-70B linears at M = 1: qkv, 640 tiles, 19.2 -> 17.0 us with 4 waves instead
  // of 8; down, 512 tiles, 35.0 -> 47.9 us; o, 512 tiles of 64 groups, 14.7 -> 12.5 us).  From
  // two tokens on, the staged activations cost as much L2 traffic as the weights they meet,
  // so four tiles share one staged slice (measured on the Llama-3-70B linears: at M = 8 the
  // gate_up launch drops from 147 to 79 us, at M = 5 from 87 to 71 us).
  if (M > 1) {
    p.nt = 4;
    p.waves = 2;
    // Except for a few tokens on linears of at most 128 groups: there every tile still streams
    // alone with 4 waves, as at one token (measured on the Llama-3-70B linears: qkv 19.6 ->
    // 14.6, 19.7 -> 16.3, 19.7 -> 16.7 us at M = 2, 3, 4; o 15.0 -> 12.7, 15.0 -> 13.7,
    // 15.1 -> 13.9; gate_up, 3584 tiles, 57.2 -> 51.4 at M = 2 but slower from M = 3; the
    // 224-group down no faster at M = 2 and slower above).
    if (G <= 128 && (M == 2 || (M <= 4 && p.tiles < 2048))) {
      p.nt = 1;
      p.waves = 4;
    } else if (G <= 128 && M <= 7 && p.tiles >= 640 && p.tiles < 2048) {
      // qkv-sized: four waves per tile up to seven tokens (19.98 -> 17.93, 20.04 -> 19.02,
      // 20.36 -> 19.71 us at M = 5, 6, 7; 20.65 -> 22.13 at M = 8; o-sized, 512 tiles, slower).
      p.waves = 4;
    }
  } else {
    p.nt = 1;
    p.waves = p.tiles >= 640 ? 4 : p.tiles >= 384 ? (G >= 16 * 8 ? 8 : 4) : 16;
  }
  if (int e = t(QV_TUNE_W4A8_NT)) p.nt = e >= 4 ? 4 : e >= 2 ? 2 : 1;
  if (int e = t(QV_TUNE_W4A8_WAVES)) p.waves = e;
  while (p.nt > 1 && p.tiles % p.nt != 0) p.nt /= 2;
  // Instantiated (NT, NWT): (1, 4), (1, 8), (1, 16), (2, 4), (4, 2), (4, 4).
  if (p.nt == 4) p.waves = p.waves >= 4 ? 4 : 2;
  else if (p.nt == 2) p.waves = 4;
  else p.waves = p.waves >= 16 ? 16 : p.waves >= 8 ? 8 : 4;
  while (p.waves > 4 && p.nt == 1 && G < p.waves) p.waves /= 2;
  // K is split until there are about 2048 waves at M = 1, 4096 from two tokens on (measured
  // on the Llama-3-70B linears at M = 5, four-tile workgroups: down 44.5 -> 38.3 us, o 17.9 ->
  // 16.7 us, qkv 22.6 -> 21.6 us with 4 splits instead of 2).
  const int wgs = p.tiles / p.nt, nw = p.nt * p.waves;
  const int wave_target = M > 1 ? 4096 : 2048;
  int splits = 1;
  if (wgs * nw < wave_target) splits = (wave_target + wgs * nw - 1) / (wgs * nw);
  const int max_splits = G / p.waves > 0 ? G / p.waves : 1;  // at least one group per wave
  if (splits > max_splits) splits = max_splits;
  // At least two batches of the weight ring (16 groups) per wave where splitting less still
  // leaves every wave that many (measured at M = 5: qkv 20.9 -> 19.9 us and o 16.5 -> 15.3 us
  // with 2 splits instead of 4).
  while (splits > 1 && G / (splits * p.waves) < 2 * kP) --splits;
  if (int e = t(QV_TUNE_W4A8_SPLITS)) splits = e;
  if (splits < 1) splits = 1;
  if (splits > G) splits = G;
  int gps = (G + splits - 1) / splits;
  const int lds_kb = t(QV_TUNE_W4A8_LDS_KB);
  const size_t lds_max = lds_kb ? (size_t)lds_kb * 1024 : kLdsMax;
  while (gps > 1 && lds_layout(M, gps, p.nt).total > lds_max) --gps;
  splits = (G + gps - 1) / gps;
  if (wgs > QV_WORKSPACE_COUNTER_BYTES / 4) splits = 1, gps = G;  // (not reached for N < 2^18)
  p.splits = splits;
  p.k_per_split = gps * kGroup;
  p.variant = (M + 15) / 16;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
  // The staged slice must fit in LDS (only a shape past the counter region's 16384 tile
  // blocks, forced to one split, could exceed it).
  p.ok = lds_layout(M, gps, p.nt).total <= 156 * 1024;
  return p;
}

hipError_t launch_w4a8(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                       const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                       uint16_t* y, unsigned* counters, void* partials, hipStream_t stream) {
#define QV_W4A8_CHUNK(MT)                                                                     \
  case 16 + MT:                                                                              \
    if (p.nt == 10)                                                                          \
      return p.waves == 8 ? launch_chunk<MT, 10, 8>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream)              \
                          : launch_chunk<MT, 10, 4>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream);             \
    if (p.nt == 14)                                                                          \
      return p.waves == 8 ? launch_chunk<MT, 14, 8>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream)              \
                          : launch_chunk<MT, 14, 4>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream);             \
    if (p.nt == 16)                                                                          \
      return p.waves == 8 ? launch_chunk<MT, 16, 8>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream)              \
                          : launch_chunk<MT, 16, 4>(p, xq, sx, M, K, qw, scales, zeros, N, y,  \
                                                    counters, partials, stream);             \
    return p.waves == 8 ? launch_chunk<MT, 8, 8>(p, xq, sx, M, K, qw, scales, zeros, N, y,     \
                                                 counters, partials, stream)                 \
                        : launch_chunk<MT, 8, 4>(p, xq, sx, M, K, qw, scales, zeros, N, y,     \
                                                 counters, partials, stream);
  switch (p.variant) {
    QV_W4A8_CHUNK(2)
    QV_W4A8_CHUNK(3)
    QV_W4A8_CHUNK(4)
#undef QV_W4A8_CHUNK
    case 1: return launch_m<1>(p, xq, sx, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 2: return launch_m<2>(p, xq, sx, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 3: return launch_m<3>(p, xq, sx, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    case 4: return launch_m<4>(p, xq, sx, M, K, qw, scales, zeros, N, y, counters, partials, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qv
