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
  // Pin the fp32 rounding of the second product.  Without this opaque step the compiler
  // folds the product and the fp16 conversion into v_fma_mixlo_f16, which rounds once
  // (to fp16) instead of twice and so differs from the definition in about 1 of 20000 outputs.
  asm("" : "+v"(t));
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
  // Epilogue scales, fetched now so the epilogue does not wait on a global load.  Thread
  // t owns outputs t, t + NW*64, ... of the MT*256 in the tile (token j, channel i).
  constexpr int EPT = (MT * 256 + NW * 64 - 1) / (NW * 64);
  float esx[EPT], esw[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int m = min((t >> 8) * 16 + ((t >> 4) & 15), M - 1);
    esx[k] = t < MT * 256 ? sx[m] : 0.f;
    esw[k] = t < MT * 256 ? sw[n0 + (t & 15)] : 0.f;
  }
  // Activations through a buffer resource over x_q (M * K bytes).  Token columns past M get
  // an offset beyond the resource, which returns zeros without reading memory, so padding M
  // up to the MFMA's 16 columns costs no load bandwidth (at M = 8 half of the B-fragment
  // bytes used to be copies of the last row).
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(xq), (short)0, M * K, 0x00020000);
  uint32_t xoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xoff[mt] = mt * 16 + r < M ? (uint32_t)((mt * 16 + r) * K + kg * 16) : 0x80000000u;

  i32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = i32x4{0, 0, 0, 0};

  // Batches of U steps; a partial last batch clamps its addresses to the wave's last step
  // (those loads hit in cache) and skips their MFMAs, so every batch issues all of its
  // loads before the first MFMA waits on one.
  for (int s = s0; s < s1; s += U) {
    i32x4 a[U];
    i32x4 b[MT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t off = (size_t)min(s + u, s1 - 1) * 64;
      a[u] = *reinterpret_cast<const i32x4*>(wp + off);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        b[mt][u] = __builtin_bit_cast(
            i32x4, __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[mt] + (uint32_t)off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u >= s1) break;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], b[mt][u], acc[mt], 0, 0, 0);
    }
  }

  // Sum the waves' tiles through LDS.  The 16x16 accumulator tile puts output (i, j) with
  // i = 4*(l/16) + v (weight row), j = l%16 (token) in lane l, register v; store it as
  // red[wave][mt][j][i] so that consecutive threads of the reduction own consecutive n.
  __shared__ int32_t red[NW][MT][16][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<i32x4*>(&red[wave][mt][r][kg * 4]) = acc[mt];
  __syncthreads();

#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int mt = t >> 8, j = (t >> 4) & 15, i = t & 15;
    const int m = mt * 16 + j;
    if (t >= MT * 256 || m >= M) continue;
    int32_t sum = 0;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) sum += red[wv][mt][j][i];
    const int n = n0 + i;
    if (splits == 1) {
      y[(size_t)m * N + n] = dequant_epilogue(sum, esx[k], esw[k]);
      if (acc_out) acc_out[(size_t)m * N + n] = sum;
    } else {
      st_coherent(&part[((size_t)split * M + m) * N + n], sum);
    }
  }
  if (splits == 1) return;

  // Split-K: the last workgroup of this tile adds the partial sums.
  if (!arrive_last(&counters[tile], (unsigned)splits)) return;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int mt = t >> 8, j = (t >> 4) & 15, i = t & 15;
    const int m = mt * 16 + j;
    if (t >= MT * 256 || m >= M) continue;
    const int n = n0 + i;
    // Loads of eight splits in flight before any is added (int32: order-free, exact).
    int32_t sum = 0;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      int32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ld_coherent(&part[((size_t)min(sp0 + j, splits - 1) * M + m) * N + n]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (sp0 + j < splits) sum += v[j];
    }
    y[(size_t)m * N + n] = dequant_epilogue(sum, esx[k], esw[k]);
    if (acc_out) acc_out[(size_t)m * N + n] = sum;
  }
}

// Ring variant: the split's x_q slice (all M rows) is staged into LDS once (by each wave for
// its own K-range when the workgroup has one tile, else by the workgroup behind one barrier),
// so the main loop's only global loads are the weights.  A workgroup owns NT
// adjacent 16-channel tiles that share the staged slice (NWT waves per tile), which divides
// the LDS footprint and the staging reads per tile by NT.  Each wave keeps the next P
// K-steps of its 16 weight rows in flight in a register ring and refills a slot as soon as
// the step in it has been consumed; the activations come from LDS (lgkmcnt), so waiting for
// them never waits for weight prefetches (vmcnt completes in order).  LDS rows are
// XOR-swizzled by 16-byte column so that the 16 token rows read at one column hit distinct
// banks.  After the main loop the same LDS holds the waves' accumulators for the exact
// int32 reduction; the epilogue is that of w8a8_kernel.
template <int MT, int NT, int NWT, int P>
__global__ __launch_bounds__(NT * NWT * 64) void w8a8_ring_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, int M, int K,
    const int8_t* __restrict__ w, const float* __restrict__ sw, int N,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, unsigned* __restrict__ counters,
    int32_t* __restrict__ part, int splits, int steps_per_split, int vpr) {
  constexpr int NW = NT * NWT;
  extern __shared__ i32x4 xs8[];  // [M][vpr] 16-byte vectors, later [NW][MT][16][16] int32
  const int group = blockIdx.x;  // NT tiles: channels 16*NT*group ..
  const int split = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int kg = lane >> 4;
  const int wt = wave % NWT;  // this wave's part of its tile's K-slice
  const int n0 = (group * NT + wave / NWT) * 16;

  const int steps_total = K >> 6;
  const int sb = split * steps_per_split;
  const int se = min(sb + steps_per_split, steps_total);
  const int ns = se - sb;
  // Waves take whole quads of 4 steps (the LDS swizzle period), the tile's last wave also
  // the leftover steps, so step phases within a quad are compile-time constants below.
  const int nq = ns >> 2;
  const int s0 = sb + 4 * ((nq * wt) / NWT);
  const int s1 = wt == NWT - 1 ? se : sb + 4 * ((nq * (wt + 1)) / NWT);

  const int8_t* wp = w + (size_t)(n0 + r) * K + kg * 16;
  // Epilogue scales, fetched now so the epilogue does not wait on a global load.  Thread
  // t owns outputs t, t + NW*64, ... of the NT*MT*256 in the workgroup: tile t / (MT*256),
  // then token j and channel i as in w8a8_kernel.
  constexpr int OUT = NT * MT * 256;
  constexpr int EPT = (OUT + NW * 64 - 1) / (NW * 64);
  float esx[EPT], esw[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int u = t % (MT * 256);
    const int m = min((u >> 8) * 16 + ((u >> 4) & 15), M - 1);
    esx[k] = t < OUT ? sx[m] : 0.f;
    esw[k] = t < OUT ? sw[(group * NT + t / (MT * 256)) * 16 + (u & 15)] : 0.f;
  }
  i32x4 wq[P];
  auto load_ring = [&]() {
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (s0 + p < s1) wq[p] = *reinterpret_cast<const i32x4*>(wp + (size_t)(s0 + p) * 64);
  };

  // Stage x_q[:, 64*sb .. 64*se) into LDS, 8 loads in flight per thread per round; vectors
  // past the end load the last one (a cache hit) and are not stored.  The first round's
  // staging loads (L2 hits) go out before the weight ring (HBM), so the first stores need not
  // wait for the whole ring (measured on the 12288-deep down projection at M = 8: 14.35 ->
  // 14.20 us).  The compiled waits count the staging loads only (the ring's loads are
  // conditional), so the round's last store still waits for the ring; with the ring's loads
  // unconditional (clamped), the stores wait for the staging loads alone, which measured
  // level on gate_up and the LM head and 3 % slower on the down projection.
  if constexpr (NT == 1) {
    // One tile per workgroup: the waves' K-ranges are disjoint, so each wave stages just the
    // columns it reads itself (its M x vw block, vw = 4 (s1 - s0) vectors per row) and needs
    // no workgroup barrier before its MFMAs: the LDS operations of one wave complete in order
    // (measured on the down projection, 16 waves per tile: 14.18 -> 13.70 us at M = 8,
    // 13.12 -> 12.65 us at M = 1).  Lane l takes the vectors e = l, l + 64, ...; each
    // position follows from the previous one by adding 64 vectors as (rows, vectors) with one
    // carry.  The block starts at a multiple of 16 vectors (waves take whole quads of steps),
    // so the swizzle keeps every vector inside the wave's own block.
    const int vw = 4 * (s1 - s0);
    const int vb = 4 * (s0 - sb);
    const int nw = M * vw;
    if (vw > 0) {
      const int dm = 64 / vw, dv = 64 - dm * vw;
      int pm = lane / vw, pv = lane - (lane / vw) * vw;
      i32x4 d[8];
      int mj[8], vj[8];
      auto load_round = [&]() {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          mj[j] = pm;
          vj[j] = pv;
          const int mc = pm < M ? pm : M - 1, vc = pm < M ? pv : vw - 1;
          d[j] = *reinterpret_cast<const i32x4*>(xq + (size_t)mc * K + (size_t)s0 * 64 + vc * 16);
          pm += dm;
          pv += dv;
          if (pv >= vw) {
            pv -= vw;
            ++pm;
          }
        }
      };
      auto store_round = [&]() {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (mj[j] < M) xs8[mj[j] * vpr + ((vb + vj[j]) ^ (mj[j] & 15))] = d[j];
      };
      load_round();
      load_ring();
      store_round();
      for (int e0 = lane + 8 * 64; e0 < nw; e0 += 8 * 64) {
        load_round();
        store_round();
      }
    } else {
      load_ring();  // a wave without steps (loads nothing)
    }
    // Only keeps the compiler from moving LDS accesses across the hand-over.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    // Several tiles share every column: the workgroup stages the slice together.  Thread t
    // takes the vectors e = t, t + NW*64, ... of the M x vrow slice.  The offsets j*NW*64 as
    // (rows, vectors) are workgroup-uniform (scalar) and each vector's position follows from
    // the thread's first one with one carry, so there is one division per thread instead of
    // two per vector (a runtime division is a long VALU sequence on the path to the first
    // MFMA) and the eight addresses do not depend on each other.
    const int vrow = ns * 4;  // 16-byte vectors per row in this split
    const int nvec = M * vrow;
    constexpr int NTHR = NW * 64;
    int jm[9], jv[9];  // (rows, vectors) of j * NTHR vectors, j = 0..8
    jm[0] = 0;
    jv[0] = 0;
    {
      const int dm = NTHR / vrow, dv = NTHR - dm * vrow;
#pragma unroll
      for (int j = 1; j <= 8; ++j) {
        jm[j] = jm[j - 1] + dm;
        jv[j] = jv[j - 1] + dv;
        if (jv[j] >= vrow) {
          jv[j] -= vrow;
          ++jm[j];
        }
      }
    }
    int m0 = (int)threadIdx.x / vrow, v0 = (int)threadIdx.x - m0 * vrow;
    i32x4 d[8];
    int mj[8], vj[8];
    auto load_round = [&]() {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int c = v0 + jv[j] >= vrow;
        mj[j] = m0 + jm[j] + c;
        vj[j] = v0 + jv[j] - c * vrow;
        const int mc = mj[j] < M ? mj[j] : M - 1, vc = mj[j] < M ? vj[j] : vrow - 1;
        d[j] = *reinterpret_cast<const i32x4*>(xq + (size_t)mc * K + (size_t)sb * 64 + vc * 16);
      }
      const int c = v0 + jv[8] >= vrow;
      m0 += jm[8] + c;
      v0 += jv[8] - c * vrow;
    };
    auto store_round = [&]() {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (mj[j] < M) xs8[mj[j] * vpr + (vj[j] ^ (mj[j] & 15))] = d[j];
    };
    int e0 = threadIdx.x;
    const bool staged = e0 < nvec;
    if (staged) load_round();
    load_ring();
    if (staged) store_round();
    for (e0 += 8 * NTHR; e0 < nvec; e0 += 8 * NTHR) {
      load_round();
      store_round();
    }
    __syncthreads();
  }

  // LDS vector index of this lane's B fragment for step st: boff[mt][(st - sb) & 3] +
  // 16 * ((st - sb) >> 2); the swizzle only permutes the 16 vectors of 4 steps.
  int boff[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) boff[mt][q] = m * vpr + ((q * 4 + kg) ^ (m & 15));
  }

  i32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = i32x4{0, 0, 0, 0};

  static_assert(P % 4 == 0, "P is a multiple of 4 steps");
  // Consume slot p, then refill it with the step P later.  (Measured: making these loads
  // unconditional with clamped steps, so the compiler could wait for single loads, made the
  // kernel 10-16% slower here; the ring is drained once per P steps instead.)
  for (int s = s0; s < s1; s += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int st = s + p;
      if (st < s1) {
        const int quad = ((s - sb) >> 2) + (p >> 2);  // (s - sb) and P are multiples of 4
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wq[p], xs8[boff[mt][p & 3] + 16 * quad],
                                                          acc[mt], 0, 0, 0);
        if (st + P < s1) wq[p] = *reinterpret_cast<const i32x4*>(wp + (size_t)(st + P) * 64);
      }
    }
  }

  // Every wave is done reading the staged slice before the accumulators overwrite it.
  __syncthreads();
  int32_t(*red)[MT][16][16] = reinterpret_cast<int32_t(*)[MT][16][16]>(xs8);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<i32x4*>(&red[wave][mt][r][kg * 4]) = acc[mt];
  __syncthreads();

#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int it = t / (MT * 256), u = t % (MT * 256);
    const int mt = u >> 8, j = (u >> 4) & 15, i = u & 15;
    const int m = mt * 16 + j;
    if (t >= OUT || m >= M) continue;
    int32_t sum = 0;
#pragma unroll
    for (int wv = 0; wv < NWT; ++wv) sum += red[it * NWT + wv][mt][j][i];
    const int n = (group * NT + it) * 16 + i;
    if (splits == 1) {
      y[(size_t)m * N + n] = dequant_epilogue(sum, esx[k], esw[k]);
      if (acc_out) acc_out[(size_t)m * N + n] = sum;
    } else {
      st_coherent(&part[((size_t)split * M + m) * N + n], sum);
    }
  }
  if (splits == 1) return;
  if (!arrive_last(&counters[group], (unsigned)splits)) return;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int t = threadIdx.x + k * NW * 64;
    const int it = t / (MT * 256), u = t % (MT * 256);
    const int mt = u >> 8, j = (u >> 4) & 15, i = u & 15;
    const int m = mt * 16 + j;
    if (t >= OUT || m >= M) continue;
    const int n = (group * NT + it) * 16 + i;
    // Loads of eight splits in flight before any is added (int32: order-free, exact).
    int32_t sum = 0;
    for (int sp0 = 0; sp0 < splits; sp0 += 8) {
      int32_t v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = ld_coherent(&part[((size_t)min(sp0 + j, splits - 1) * M + m) * N + n]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (sp0 + j < splits) sum += v[j];
    }
    y[(size_t)m * N + n] = dequant_epilogue(sum, esx[k], esw[k]);
    if (acc_out) acc_out[(size_t)m * N + n] = sum;
  }
}

// LDS the ring kernel needs: the staged x_q slice (row length rounded up to 16 vectors so
// the XOR swizzle stays inside the row), or the waves' accumulators if those are larger.
size_t ring_lds_bytes(int M, int steps_per_split, int waves) {
  const int vpr = ((steps_per_split * 4 + 15) / 16) * 16;
  const size_t xs = (size_t)M * vpr * sizeof(i32x4);
  const size_t red = (size_t)waves * ((M + 15) / 16) * 256 * sizeof(int32_t);
  return xs > red ? xs : red;
}
constexpr size_t kRingLdsMax = 128 * 1024;

// Ring depth P (K-steps in flight per lane), chosen by the planner: for 4-wave tiles, one or
// two per workgroup, 16 with more than one token (measured on the Qwen3-8B shapes: at M = 8
// one tile per workgroup, gate_up 24.7 -> 23.9 us, LM head 128.7 -> 123.9 us; at M = 10 two
// tiles, gate_up 25.3 -> 24.4 us, LM head 133.4 -> 128.6 us), 8 otherwise (at M = 1 the LM
// head, and at M = 8 the 16-wave down projection, are faster with 8); for 2-wave tiles see
// plan_w8a8.
template <int MT, int NT, int NWT, int P = 8>
hipError_t launch_ring(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                       const int8_t* w, const float* sw, int N, uint16_t* y, int32_t* acc_out,
                       unsigned* counters, void* partials, hipStream_t stream) {
  // The grid covers tiles / NT workgroups: a tile count NT does not divide would leave
  // channels unwritten, so it is refused rather than launched.
  if (p.tiles % NT != 0) return hipErrorInvalidValue;
  const int sps = p.k_per_split / 64;
  const int vpr = ((sps * 4 + 15) / 16) * 16;
  const size_t lds = ring_lds_bytes(M, sps, NT * NWT);
  auto kern = w8a8_ring_kernel<MT, NT, NWT, P>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.tiles / NT, p.splits);
  kern<<<grid, NT * NWT * 64, lds, stream>>>(xq, sx, M, K, w, sw, N, y, acc_out, counters,
                                            static_cast<int32_t*>(partials), p.splits, sps, vpr);
  return hipGetLastError();
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

GemmPlan plan_w8a8(int M, int N, int K, const Tuning& t) {
  GemmPlan p{};
  p.tiles = N / 16;
  const int steps = K / 64;
  // Keep every CU streaming with no cross-workgroup traffic: one workgroup per 16-channel
  // tile, and enough waves per workgroup (4, 8 or 16, all splitting the tile's K) that the
  // launch keeps every CU busy: with >= 1024 tiles 2 waves, 8 from 384, else 16 (measured
  // best on the Qwen3-8B and LM-head shapes; at M = 1 the 2-wave tiles take gate_up from 21.5
  // to 20.4 us against 4-wave ones, the LM head from 109.7 to 111.7 us).  Only when even 16
  // waves per tile cannot provide about 2048 waves is K split across workgroups as well.
  p.waves = p.tiles >= 1024 ? 2 : p.tiles >= 384 ? 8 : 16;
  while (p.waves > 4 && steps < 2 * p.waves) p.waves /= 2;
  if (int e = t(QV_TUNE_W8A8_WAVES)) p.waves = e >= 16 ? 16 : e >= 8 ? 8 : e >= 4 ? 4 : 2;
  int splits = 1;
  if (p.tiles * p.waves < 2048) {
    splits = (2048 + p.tiles * p.waves - 1) / (p.tiles * p.waves);
    const int max_splits = steps / (2 * p.waves) > 0 ? steps / (2 * p.waves) : 1;
    if (splits > max_splits) splits = max_splits;
  }
  if (int e = t(QV_TUNE_W8A8_SPLITS)) splits = e;
  if (splits > steps) splits = steps;
  if (splits < 1) splits = 1;
  if (p.tiles > QV_WORKSPACE_COUNTER_BYTES / 4) splits = 1;
  const int steps_per_split = (steps + splits - 1) / splits;
  splits = (steps + steps_per_split - 1) / steps_per_split;
  p.splits = splits;
  p.k_per_split = steps_per_split * 64;
  p.variant = (M + 15) / 16;
  // The LDS-staged ring kernel (variant + 8) for many tiles or long K, where it streams
  // 15-25% faster; the direct kernel for the few-tile, short-K shapes, where the staging
  // prologue does not pay off.  Either way only when the staged slice fits in LDS.
  bool ring = p.tiles >= 1024 || K >= 8192;
  if (int e = t(QV_TUNE_W8A8_RING)) ring = e == 1;
  // Tiles per ring workgroup: they share one staged slice, so more of them divide the LDS
  // footprint per tile, letting more tiles stay resident per CU.  Two 2-wave tiles per
  // workgroup with a 16-step ring (measured on the Qwen3-8B shapes against one 4-wave tile:
  // gate_up 24.3 -> 22.2 us at M = 8 and 24.4 -> 23.1 us at M = 10, the LM head 128.9 ->
  // 121.2 us at M = 8) fit a whole gate_up launch (768 workgroups of 32 KB of LDS) on the
  // chip at once, where 1536 single-tile workgroups needed a second, partial round.  With
  // 4-wave tiles (only by override) two tiles per workgroup above M = 8.
  p.nt = p.waves == 2 || (M > 8 && p.waves == 4) ? 2 : 1;
  if (int e = t(QV_TUNE_W8A8_NT)) p.nt = e >= 4 ? 4 : e >= 2 ? 2 : 1;
  while (p.nt > 1 && (p.tiles % p.nt != 0 || p.waves * p.nt > 16)) p.nt /= 2;
  if (ring_lds_bytes(M, steps_per_split, p.waves * p.nt) > kRingLdsMax) ring = false;
  if (ring) {
    p.variant += 8;
  } else {
    p.nt = 1;
    if (p.waves < 4) p.waves = 4;
  }
  // Ring depth.  4-wave tiles: 16 K-steps with more than one token and one or two tiles per
  // workgroup, else 8.  2-wave tiles: 8 (111 VGPRs, 4 waves per SIMD, against 143 and 3 with
  // 16: measured on the Qwen3-8B verify step at M = 8, the gate_up/LM-head launches 23.27 ->
  // 22.76 us on average and the step 2.446 -> 2.426 ms; only the 151936-channel LM head alone
  // is faster with 16, 116.1 against 118.4 us).
  p.ring = p.nt <= 2 && M > 1 ? 16 : 8;
  if (p.waves == 2) p.ring = 8;
  // 16-wave tiles (the 12288-deep down projection: 12 K-steps per wave): 12, each wave's
  // whole slice in flight at 126 VGPRs (still 4 waves per SIMD); 2 % faster than 8 at M = 1..8.
  if (p.waves == 16) p.ring = 12;
  if (int e = t(QV_TUNE_W8A8_RINGP)) p.ring = e >= 16 ? 16 : e >= 12 ? 12 : 8;
  p.partial_bytes = splits > 1 ? (size_t)splits * M * N * sizeof(int32_t) : 0;
  p.ok = true;  // every shape of the rules has a plan (the direct kernel needs no LDS budget)
  return p;
}

hipError_t launch_w8a8(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                       const int8_t* w, const float* sw, int N, uint16_t* y, int32_t* acc_out,
                       unsigned* counters, void* partials, hipStream_t stream) {
#define QV_W8A8_ARGS p, xq, sx, M, K, w, sw, N, y, acc_out, counters, partials, stream
#define QV_W8A8_CASE(MT, U)                                            \
  case MT:                                                             \
    if (p.waves == 16) return launch_t<MT, U, 16>(QV_W8A8_ARGS);       \
    if (p.waves == 8) return launch_t<MT, U, 8>(QV_W8A8_ARGS);         \
    return launch_t<MT, U, 4>(QV_W8A8_ARGS);
#define QV_W8A8_RING(MT)                                                       \
  case 8 + MT:                                                                 \
    if (p.waves == 16)                                                         \
      return p.ring == 12 ? launch_ring<MT, 1, 16, 12>(QV_W8A8_ARGS)           \
                          : launch_ring<MT, 1, 16>(QV_W8A8_ARGS);              \
    if (p.waves == 8)                                                          \
      return p.nt == 2 ? launch_ring<MT, 2, 8>(QV_W8A8_ARGS)                   \
                       : launch_ring<MT, 1, 8>(QV_W8A8_ARGS);                  \
    if (p.waves == 2) {                                                        \
      /* tiles per workgroup from p.nt in every arm (the grid is tiles / NT) */ \
      if (p.nt == 4) return launch_ring<MT, 4, 2, 16>(QV_W8A8_ARGS);           \
      if (p.nt == 2)                                                           \
        return p.ring == 8    ? launch_ring<MT, 2, 2, 8>(QV_W8A8_ARGS)         \
               : p.ring == 12 ? launch_ring<MT, 2, 2, 12>(QV_W8A8_ARGS)        \
                              : launch_ring<MT, 2, 2, 16>(QV_W8A8_ARGS);       \
      return p.ring == 8 ? launch_ring<MT, 1, 2, 8>(QV_W8A8_ARGS)              \
                         : launch_ring<MT, 1, 2, 16>(QV_W8A8_ARGS);            \
    }                                                                          \
    if (p.nt == 4)                                                             \
      return p.ring == 16 ? launch_ring<MT, 4, 4, 16>(QV_W8A8_ARGS)            \
                          : launch_ring<MT, 4, 4>(QV_W8A8_ARGS);               \
    if (p.nt == 2)                                                             \
      return p.ring == 16 ? launch_ring<MT, 2, 4, 16>(QV_W8A8_ARGS)            \
                          : launch_ring<MT, 2, 4>(QV_W8A8_ARGS);               \
    return p.ring == 16 ? launch_ring<MT, 1, 4, 16>(QV_W8A8_ARGS)              \
                        : launch_ring<MT, 1, 4>(QV_W8A8_ARGS);
  switch (p.variant) {
    QV_W8A8_CASE(1, 8)
    QV_W8A8_CASE(2, 4)
    QV_W8A8_CASE(3, 2)
    QV_W8A8_CASE(4, 2)
    QV_W8A8_RING(1)
    QV_W8A8_RING(2)
    QV_W8A8_RING(3)
    QV_W8A8_RING(4)
    default:
      return hipErrorInvalidValue;
  }
#undef QV_W8A8_RING
#undef QV_W8A8_CASE
#undef QV_W8A8_ARGS
}

}  // namespace qv
