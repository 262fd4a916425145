// Stochastic verification at temperature T > 0 (Quasar, Sec. 3.3 "Lossless Rejection
// Sampling": the target distribution p, recovered in high precision, is compared with the
// draft distribution q; Sec. 2.1 and the speculative-sampling abstract of the search-results
// page name the modified rejection sampling of speculative decoding, which is what is built
// here).  Every probability is computed in float64.
//
// Two launches on the caller's stream:
//
//  1. sample_stats_kernel, a grid of (chunks x rows) workgroups over the target rows and,
//     when given, the drafter's rows, each reducing one chunk of one row to (chunk maximum,
//     sum of exp((x - chunk maximum) / T)), and recording the logit of the row's draft token.
//     No workgroup waits for another.
//  2. sample_draw_kernel, a grid over 2048-logit chunks.  Every workgroup stages all chunk
//     statistics in LDS, combines them into each row's maximum and softmax denominator, takes
//     the acceptance tests (draft i is accepted iff u[i] * q_i(x_i) < p_i(x_i)) and finds the
//     first rejection, all redundantly and identically; then it sums the weights of its
//     chunk of the emitting row: max(0, p - q) for a rejected row, p for the bonus row.  The
//     last workgroup to arrive locates u[M-1] times the total in the running sums, first the
//     chunk, then the element, with block-wide prefix scans.
//
// The results agree with a sequential float64 evaluation except where a decision lies
// within a few units in the last place of a tie (the summation orders differ).
#include <math.h>

#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kStep1 = 4096;     // logits per statistics-pass iteration (16 per thread)
constexpr int kMaxChunks1 = 64;  // statistics chunks per row (bounds the draw's staging)
constexpr int kChunk2 = 2048;    // logits per workgroup of the draw (8 per thread)
constexpr int kDrawCounter = 255;
constexpr int kStoreMaxV = 1 << 20;  // the draw keeps per-logit weights up to this vocabulary

typedef double f64x2 __attribute__((ext_vector_type(2)));

struct SampleArgs {
  const uint16_t* logits;   // target [M][V]
  const uint16_t* dlogits;  // drafter [M-1][V], or null for a point-mass drafter
  const int32_t* draft;     // [M-1]
  const double* u;          // [M]
  double T, invT;           // temperature and its correctly rounded reciprocal
  int M, V, rows;           // rows = M + (dlogits ? M - 1 : 0)
  int group;                // lanes per row when the draw kernel combines row statistics
  int chunk1;               // logits per statistics chunk (a multiple of kStep1)
  int chunks1, chunks2;
  int32_t* result;          // {n_accept, token}
  unsigned* counter;
  double* part1;            // [rows][chunks1][2]  (chunk maximum, sum of exp)
  double* xlogit;           // [rows]              logit of the row's draft token
  uint64_t* part2;          // [chunks2][kWaves][2] per-wave (weight sum, p sum), float64 bits
  uint64_t* wbuf;           // [chunks2 * kChunk2]  per-logit draw weights, or null (recompute)
};

__device__ __forceinline__ double h2d(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint64_t dbits(double d) { return __builtin_bit_cast(uint64_t, d); }
__device__ __forceinline__ double bitsd(uint64_t b) { return __builtin_bit_cast(double, b); }

__device__ __forceinline__ const uint16_t* row_ptr(const SampleArgs& a, int r) {
  return r < a.M ? a.logits + (size_t)r * a.V : a.dlogits + (size_t)(r - a.M) * a.V;
}

// Index into draft[] of row r's token (target row r < M-1 verifies draft[r], drafter row
// M + i proposes draft[i]); -1 for the bonus row.
__device__ __forceinline__ int draft_index(const SampleArgs& a, int r) {
  return r < a.M - 1 ? r : (r >= a.M ? r - a.M : -1);
}

__device__ __forceinline__ void decode8(u32x4 d, double (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = h2d((uint16_t)(d[j] & 0xFFFFu));
    x[2 * j + 1] = h2d((uint16_t)(d[j] >> 16));
  }
}

// Eight consecutive logits starting at element e as float64; positions at or past V are
// -inf.  One 16-byte load when the row allows it.
__device__ __forceinline__ void load8(const uint16_t* row, long e, int V, bool vec, double (&x)[8]) {
  if (vec && e + 8 <= V) {
    decode8(*reinterpret_cast<const u32x4*>(row + e), x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = e + j < V ? h2d(row[e + j]) : -INFINITY;
  }
}

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Block-wide max / sum; every thread gets the result.  `sh` holds kWaves doubles.
__device__ __forceinline__ double block_max_d(double v, double* sh) {
  v = wave_max_d(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmax(r, sh[i]);
  return r;
}
__device__ __forceinline__ double block_sum_d(double v, double* sh) {
  v = wave_sum_d(v);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r += sh[i];
  return r;
}

// Prefix sums over the block in thread order: returns the inclusive sum and sets `excl` to
// the exclusive one (both accumulate the same partial sums).  `sh` holds kWaves doubles.
__device__ __forceinline__ double block_scan_d(double v, double* sh, double& excl) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  const double prev = __shfl_up(v, 1, kWave);
  __syncthreads();
  if (lane == kWave - 1) sh[wave] = v;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < wave; ++i) base += sh[i];
  excl = lane ? base + prev : base;
  return base + v;
}

// Lowest thread index whose predicate holds, or -1; uniform across the block.
__device__ __forceinline__ int block_first(bool pred, int* sh) {
  const uint64_t m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = m ? (int)__builtin_ctzll(m) : -1;
  __syncthreads();
  for (int i = 0; i < kWaves; ++i)
    if (sh[i] >= 0) return i * kWave + sh[i];
  return -1;
}
// Highest thread index whose predicate holds, or -1; uniform across the block.
__device__ __forceinline__ int block_last(bool pred, int* sh) {
  const uint64_t m = __ballot(pred);
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[threadIdx.x / kWave] = m ? 63 - (int)__builtin_clzll(m) : -1;
  __syncthreads();
  for (int i = kWaves - 1; i >= 0; --i)
    if (sh[i] >= 0) return i * kWave + sh[i];
  return -1;
}

// ---- pass 1: chunk statistics ----------------------------------------------------------
// Workgroup (c, r) reduces logits [c * chunk1, (c + 1) * chunk1) of row r to (m, s) with m the
// chunk maximum and s = sum exp((x - m) / T); each thread keeps a running (maximum, sum) over
// its 16-logit slices, rescaling the sum when the maximum grows.  The workgroup whose slice
// holds the row's draft token also records that logit.  Plain stores: the draw kernel reads
// them after this launch completes.
__global__ __launch_bounds__(kThreads) void sample_stats_kernel(SampleArgs a) {
  const int c = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
  __shared__ double shd[kWaves];
  const uint16_t* row = row_ptr(a, r);
  const bool vec = (a.V & 7) == 0;
  const int di = draft_index(a, r);
  const int xr = di >= 0 ? a.draft[di] : -1;

  const long beg = (long)c * a.chunk1;
  const long end = min(beg + (long)a.chunk1, (long)a.V);
  double m = -INFINITY, s = 0.0;
  for (long base = beg; base < end; base += kStep1) {
    double x[2][8];
    load8(row, base + tid * 8, a.V, vec, x[0]);
    load8(row, base + kThreads * 8 + tid * 8, a.V, vec, x[1]);
    const long o = (long)xr - base;  // the draft token's offset in this slice
    if (o >= 0 && o < kStep1 && xr < a.V && (int)((o & (kThreads * 8 - 1)) >> 3) == tid) {
      const int h = (int)(o / (kThreads * 8)), jj = (int)(o & 7);
      double v = 0.0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (hh == h && j == jj) v = x[hh][j];
      a.xlogit[r] = v;
    }
    double lm = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) lm = fmax(lm, x[h][j]);
    if (lm > m) {
      if (s > 0.0) s *= exp((m - lm) * a.invT);
      m = lm;
    }
    if (m > -INFINITY) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += exp((x[h][j] - m) * a.invT);
    }
  }
  const double cm = block_max_d(m, shd);
  const double cs = block_sum_d(m > -INFINITY ? s * exp((m - cm) * a.invT) : 0.0, shd);
  if (tid == 0) {
    double* p = a.part1 + ((size_t)r * a.chunks1 + c) * 2;
    p[0] = cm;
    p[1] = cs;
  }
}

// ---- pass 2: acceptance and the emitted token -----------------------------------------
struct DrawRow {
  const uint16_t* p_row;
  const uint16_t* q_row;  // null: point mass at xq (none if xq is outside [0, V))
  double pm, pinv, qm, qinv;  // row maximum and reciprocal softmax denominator
  int xq;
  bool residual;
};

// Two float64 values written through to the device coherence point as one 16-byte store.
__device__ __forceinline__ void st_coherent_d2(uint64_t* p, double lo, double hi) {
  st_coherent_f4(reinterpret_cast<float*>(p), __builtin_bit_cast(f32x4, f64x2{lo, hi}));
}

// Weights of the eight elements e .. e+7 from their target (and drafter) logits: p and,
// when residual, max(0, p - q); elements past V weigh 0.
__device__ __forceinline__ void weights8(const SampleArgs& a, const DrawRow& d, long e,
                                         const double (&xp)[8], const double (&xq)[8],
                                         double (&p)[8], double (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = e + j < a.V ? exp((xp[j] - d.pm) * a.invT) * d.pinv : 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    double q = 0.0;
    if (d.q_row)
      q = e + j < a.V ? exp((xq[j] - d.qm) * a.invT) * d.qinv : 0.0;
    else
      q = e + j == d.xq ? 1.0 : 0.0;
    w[j] = d.residual ? fmax(p[j] - q, 0.0) : p[j];
  }
}

// Every workgroup first combines the chunk statistics of all rows into each row's maximum
// and softmax denominator (staged through LDS in one round of loads), takes the acceptance
// tests and finds the emitting row; then it computes the weights of its 2048-logit chunk of
// that row (with PF > 0, the chunk of every row was loaded in that same first round, so the
// emitting row's logits are already in registers), and the last workgroup to arrive draws
// the token from the chunk sums and the stored per-logit weights.
template <int PF>
__global__ __launch_bounds__(kThreads) void sample_draw_kernel(SampleArgs a) {
  extern __shared__ f64x2 stage[];  // [rows][chunks1] chunk statistics, then [rows] row statistics
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  __shared__ double shd[kWaves];
  __shared__ int shi[kWaves];
  __shared__ int s_n, s_x;
  const int npairs = a.rows * a.chunks1;
  f64x2* rst = stage + npairs;
  const long e = (long)c * kChunk2 + tid * 8;
  const bool vec = (a.V & 7) == 0;

  u32x4 pre[PF > 0 ? PF : 1];
  if constexpr (PF > 0) {  // launched only with V % 8 == 0 and rows <= PF
    const long ec = e + 8 <= a.V ? e : 0;  // past V: any in-bounds slice, weighed 0 later
#pragma unroll
    for (int r = 0; r < PF; ++r)
      pre[r] = r < a.rows ? *reinterpret_cast<const u32x4*>(row_ptr(a, r) + ec) : u32x4{0, 0, 0, 0};
  }
  // The first 4 * kThreads chunk statistics, the drafts, their logits and the uniforms are
  // loaded unconditionally (indices clamped) so that every load of this first round is in
  // flight at once; larger stagings continue in a loop.
  const f64x2* src = reinterpret_cast<const f64x2*>(a.part1);
  f64x2 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = src[min(tid + k * kThreads, npairs - 1)];
  const int li = min(lane, a.M > 1 ? a.M - 2 : 0);
  const int32_t* dsrc = a.M > 1 ? a.draft : reinterpret_cast<const int32_t*>(a.u);
  const int xi = dsrc[li];
  const double xlp = a.xlogit[li];
  const double xlq = a.xlogit[a.dlogits ? a.M + li : li];
  const double ui = a.u[li];
  // (The LDS allocation holds at least 4 * kThreads entries, so these stores need no
  // condition; entries past npairs are overwritten by the row statistics later.)
#pragma unroll
  for (int k = 0; k < 4; ++k) stage[tid + k * kThreads] = v[k];
  for (int i = tid + 4 * kThreads; i < npairs; i += kThreads) stage[i] = src[i];
  __syncthreads();
  // Row r's maximum and denominator: `group` lanes per row, all rows at once.
  {
    const int G = a.group, r = tid / G, gl = tid % G;
    const f64x2* pr = stage + (size_t)r * a.chunks1;
    double m = -INFINITY;
    if (r < a.rows)
      for (int j = gl; j < a.chunks1; j += G) m = fmax(m, pr[j][0]);
    for (int off = G >> 1; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off, kWave));
    double sum = 0.0;
    if (r < a.rows)
      for (int j = gl; j < a.chunks1; j += G) {
        const f64x2 v = pr[j];
        if (v[1] > 0.0) sum += v[1] * exp((v[0] - m) * a.invT);
      }
    for (int off = G >> 1; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (r < a.rows && gl == 0) rst[r] = f64x2{m, sum};
  }
  __syncthreads();
  // Draft i (lane i of wave 0) is accepted iff u[i] * q_i(x_i) < p_i(x_i).
  if (wave == 0) {
    bool rejected = false;
    if (lane < a.M - 1) {
      rejected = true;
      if (xi >= 0 && xi < a.V) {  // lane < M - 1: xi, xlp, xlq and ui are this draft's
        const f64x2 sp = rst[lane];
        const double p = exp((xlp - sp[0]) * a.invT) / sp[1];
        double q = 1.0;
        if (a.dlogits) {
          const f64x2 sq = rst[a.M + lane];
          q = exp((xlq - sq[0]) * a.invT) / sq[1];
        }
        rejected = !(ui * q < p);
      }
    }
    const uint64_t mask = __ballot(rejected);
    const int n = mask ? (int)__builtin_ctzll(mask) : a.M - 1;
    if (lane == 0) s_n = n;
    if (lane == n) s_x = xi;
  }
  __syncthreads();
  const int n = s_n;
  if (c == 0 && tid == 0) a.result[0] = n;

  DrawRow d;
  d.residual = n < a.M - 1;
  d.p_row = a.logits + (size_t)n * a.V;
  d.pm = rst[n][0];
  d.pinv = 1.0 / rst[n][1];
  d.q_row = nullptr;
  d.qm = d.qinv = 0.0;
  d.xq = d.residual ? s_x : -1;
  if (d.residual && a.dlogits) {
    d.q_row = a.dlogits + (size_t)n * a.V;
    d.qm = rst[a.M + n][0];
    d.qinv = 1.0 / rst[a.M + n][1];
  }

  double xp[8], xq[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (PF > 0) {
    u32x4 rp = pre[0], rq = pre[0];
#pragma unroll
    for (int r = 0; r < PF; ++r) {
      if (r == n) rp = pre[r];
      if (r == a.M + n) rq = pre[r];
    }
    decode8(rp, xp);
    if (d.q_row) decode8(rq, xq);
  } else {
    load8(d.p_row, e, a.V, vec, xp);
    if (d.q_row) load8(d.q_row, e, a.V, vec, xq);
  }
  double p[8], w[8];
  weights8(a, d, e, xp, xq, p, w);
  double sw = 0.0, sp = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sw += w[j];
    sp += p[j];
  }
  sw = wave_sum_d(sw);
  sp = wave_sum_d(sp);
  if (lane == 0) st_coherent_d2(&a.part2[((size_t)c * kWaves + wave) * 2], sw, sp);
  if (a.wbuf) {
#pragma unroll
    for (int j = 0; j < 8; j += 2) st_coherent_d2(&a.wbuf[e + j], w[j], w[j + 1]);
  }
  if (!arrive_last(&a.counter[kDrawCounter], (unsigned)a.chunks2)) return;

  // Chunk level: thread t owns chunks [t * span, (t + 1) * span); a chunk's value is the
  // sum of its waves' sums in wave order.  Residual weights unless they are all zero, then p.
  const int span = (a.chunks2 + kThreads - 1) / kThreads;
  const int c0 = tid * span, c1 = min(c0 + span, a.chunks2);
  auto chunk_val = [&](int j, int which) {
    double v = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) v += bitsd(ld_coherent(&a.part2[((size_t)j * kWaves + k) * 2 + which]));
    return v;
  };
  double tw = 0.0, tp = 0.0;
  for (int j = c0; j < c1; ++j) {
    tw += chunk_val(j, 0);
    tp += chunk_val(j, 1);
  }
  const double total_w = block_sum_d(tw, shd);
  const bool use_w = d.residual && total_w > 0.0;
  const int k = use_w ? 0 : 1;
  const double mine = use_w ? tw : tp;
  double excl;
  const double incl = block_scan_d(mine, shd, excl);
  __shared__ double s_total;
  if (tid == kThreads - 1) s_total = incl;
  __syncthreads();
  const double t = a.u[a.M - 1] * s_total;

  // The chunk holding t: inside the first span whose running sum passes t, else (rounding
  // kept every running sum at or below t) the last chunk of positive weight of that span or,
  // failing that, of the row.  With one chunk per thread the span needs no second look.
  __shared__ int s_chunk;
  __shared__ double s_base;
  const int owner = block_first(incl > t, shi);
  const int who = owner >= 0 ? owner : block_last(mine > 0.0, shi);
  if (tid == 0) s_chunk = -1;
  __syncthreads();
  if (who >= 0 && tid == who) {
    if (span == 1) {
      s_chunk = c0;
      s_base = excl;
    } else {
      double run = excl;
      int found = -1, last = -1;
      double found_base = 0.0, last_base = 0.0;
      for (int j = c0; j < c1; ++j) {
        const double v = chunk_val(j, k);
        if (v > 0.0) {
          last = j;
          last_base = run;
        }
        if (found < 0 && run + v > t) {
          found = j;
          found_base = run;
        }
        run += v;
      }
      s_chunk = owner >= 0 && found >= 0 ? found : last;
      s_base = owner >= 0 && found >= 0 ? found_base : last_base;
    }
  }
  __syncthreads();
  const int cs = s_chunk;
  if (cs < 0) {  // no positive weight anywhere (non-finite logits)
    if (tid == 0) a.result[1] = -1;
    return;
  }
  const bool exact = owner >= 0;  // otherwise take the chunk's last element of positive weight

  // Element level inside chunk cs: thread t owns elements cs * kChunk2 + 8t .. 8t+7.  The
  // stored weights are those drawn from unless the residual is all zero (then p is used).
  const long ee = (long)cs * kChunk2 + tid * 8;
  double ew[8];
  if (a.wbuf && (use_w || !d.residual)) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ew[j] = bitsd(ld_coherent(&a.wbuf[ee + j]));
  } else {
    load8(d.p_row, ee, a.V, vec, xp);
    if (d.q_row) load8(d.q_row, ee, a.V, vec, xq);
    weights8(a, d, ee, xp, xq, p, w);
#pragma unroll
    for (int j = 0; j < 8; ++j) ew[j] = use_w ? w[j] : p[j];
  }
  double own = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) own += ew[j];
  const double base = s_base;
  double eexc;
  const double einc = block_scan_d(own, shd, eexc);
  const int eowner = exact ? block_first(base + einc > t, shi) : -1;
  const int ewho = eowner >= 0 ? eowner : block_last(own > 0.0, shi);
  if (tid == ewho) {
    double run = base + eexc;
    int found = -1, last = -1;
    for (int j = 0; j < 8; ++j) {
      if (ew[j] > 0.0) last = j;
      if (found < 0 && run + ew[j] > t) found = j;
      run += ew[j];
    }
    const int pick = eowner >= 0 && found >= 0 ? found : last;
    a.result[1] = pick >= 0 ? (int)(ee + pick) : -1;
  }
  if (ewho < 0 && tid == 0) a.result[1] = -1;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// Chunking of the statistics pass: 4096-logit slices, at most kMaxChunks1 chunks per row.
int chunk1_of(int V) {
  const int slices = (V + kStep1 - 1) / kStep1;
  return kStep1 * ((slices + kMaxChunks1 - 1) / kMaxChunks1);
}

// Workspace after the counters: chunk statistics [rows][chunks1][2], the draft tokens'
// logits [rows], per-wave chunk sums [chunks2][kWaves][2] and, up to kStoreMaxV logits, the
// per-logit draw weights [chunks2 * kChunk2]; each part 256-byte aligned.  Sized for the
// drafter's rows present (rows = 2M - 1).
size_t sample_partial_bytes(int M, int V) {
  const size_t rows = 2 * (size_t)M - 1;
  const int ch1 = chunk1_of(V);
  const size_t c1 = ((size_t)V + ch1 - 1) / ch1, c2 = ((size_t)V + kChunk2 - 1) / kChunk2;
  return align256(rows * c1 * 16) + align256(rows * 8) + align256(c2 * kWaves * 16) +
         (V <= kStoreMaxV ? align256(c2 * kChunk2 * 8) : 0);
}

hipError_t launch_verify_sample(const uint16_t* logits, int M, int V, const uint16_t* draft_logits,
                                const int32_t* draft, const double* uniforms, double temperature,
                                int32_t* result_out, unsigned* counters, void* partials,
                                hipStream_t stream) {
  SampleArgs a;
  a.logits = logits;
  a.dlogits = M > 1 ? draft_logits : nullptr;
  a.draft = draft;
  a.u = uniforms;
  a.T = temperature;
  a.invT = 1.0 / temperature;
  a.M = M;
  a.V = V;
  a.rows = M + (a.dlogits ? M - 1 : 0);
  a.group = 64;
  while (a.group > 1 && a.group * a.rows > kThreads) a.group >>= 1;
  a.chunk1 = chunk1_of(V);
  a.chunks1 = (V + a.chunk1 - 1) / a.chunk1;
  a.chunks2 = (V + kChunk2 - 1) / kChunk2;
  a.result = result_out;
  a.counter = counters;
  const size_t rows_max = 2 * (size_t)M - 1;
  char* base = static_cast<char*>(partials);
  a.part1 = reinterpret_cast<double*>(base);
  base += align256(rows_max * a.chunks1 * 16);
  a.xlogit = reinterpret_cast<double*>(base);
  base += align256(rows_max * 8);
  a.part2 = reinterpret_cast<uint64_t*>(base);
  base += align256((size_t)a.chunks2 * kWaves * 16);
  a.wbuf = V <= kStoreMaxV ? reinterpret_cast<uint64_t*>(base) : nullptr;

  const size_t lds = ((size_t)a.rows * a.chunks1 + a.rows > 4 * kThreads
                          ? (size_t)a.rows * a.chunks1 + a.rows
                          : 4 * kThreads) * sizeof(f64x2);
  const bool vec = (V & 7) == 0;
  auto kern = vec && a.rows <= 8    ? sample_draw_kernel<8>
              : vec && a.rows <= 16 ? sample_draw_kernel<16>
                                    : sample_draw_kernel<0>;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  sample_stats_kernel<<<dim3(a.chunks1, a.rows), kThreads, 0, stream>>>(a);
  if (hipError_t e = hipGetLastError()) return e;
  kern<<<a.chunks2, kThreads, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qv
