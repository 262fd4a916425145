// Stochastic verification at temperature T > 0 (Quasar, Sec. 3.3 "Lossless Rejection
// Sampling": the target distribution p, recovered in high precision, is compared with the
// draft distribution q; Sec. 2.1 and the speculative-sampling abstract of the search-results
// page name the modified rejection sampling of speculative decoding, which is what is built
// here).  Every probability is computed in float64.
//
// Two launches on the caller's stream:
//
//  1. sample_stats_kernel, a grid of (chunks x rows) workgroups over the target rows and,
//     when given, the drafter's rows.  Each workgroup reduces 4096 logits of one row to
//     (chunk maximum, sum of exp((x - chunk maximum) / T)).  The last workgroup of a row to
//     arrive combines the chunks into the row's maximum and softmax denominator; the last
//     row to finish takes the acceptance decisions (draft i is accepted iff
//     u[i] * q_i(x_i) < p_i(x_i)), and a wavefront ballot finds the first rejection.
//  2. sample_draw_kernel, a grid over 2048-logit chunks of the one row that emits the next
//     token: the first rejected row (weights max(0, p - q)) or the bonus row (weights p).
//     Each workgroup sums its chunk's weights; the last to arrive locates u[M-1] times the
//     total in the running sums: first the chunk, then the element, both with block-wide
//     prefix scans.
//
// The results agree with a sequential float64 evaluation except where a decision lies
// within a few units in the last place of a tie (the summation orders differ).
#include <math.h>

#include "qv_internal.h"

namespace qv {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk1 = 4096;  // logits per workgroup of the statistics pass (16 per thread)
constexpr int kChunk2 = 2048;  // logits per workgroup of the draw (8 per thread)
constexpr int kDrawCounter = 255;

struct SampleArgs {
  const uint16_t* logits;   // target [M][V]
  const uint16_t* dlogits;  // drafter [M-1][V], or null for a point-mass drafter
  const int32_t* draft;     // [M-1]
  const double* u;          // [M]
  double T;
  int M, V, rows;           // rows = M + (dlogits ? M - 1 : 0)
  int chunks1, chunks2;
  int32_t* result;          // {n_accept, token}
  unsigned* counter;
  uint64_t* part1;          // [rows][chunks1][2]  (max, sum) as float64 bits
  uint64_t* rowstat;        // [rows][2]           (max, denominator)
  int32_t* sel;             // [1]                 the emitting row
  uint64_t* part2;          // [chunks2][2]        (residual sum, p sum)
};

__device__ __forceinline__ double h2d(uint16_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ uint64_t dbits(double d) { return __builtin_bit_cast(uint64_t, d); }
__device__ __forceinline__ double bitsd(uint64_t b) { return __builtin_bit_cast(double, b); }

__device__ __forceinline__ const uint16_t* row_ptr(const SampleArgs& a, int r) {
  return r < a.M ? a.logits + (size_t)r * a.V : a.dlogits + (size_t)(r - a.M) * a.V;
}

// Eight consecutive logits starting at element e as float64; positions at or past V are
// -inf.  One 16-byte load when the row allows it.
__device__ __forceinline__ void load8(const uint16_t* row, long e, int V, bool vec, double (&x)[8]) {
  if (vec && e + 8 <= V) {
    const u32x4 d = *reinterpret_cast<const u32x4*>(row + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = h2d((uint16_t)(d[j] & 0xFFFFu));
      x[2 * j + 1] = h2d((uint16_t)(d[j] >> 16));
    }
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

// ---- pass 1: row statistics and acceptance --------------------------------------------
__global__ __launch_bounds__(kThreads) void sample_stats_kernel(SampleArgs a) {
  const int c = blockIdx.x, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  __shared__ double shd[kWaves];
  __shared__ int shi[kWaves];
  const uint16_t* row = row_ptr(a, r);
  const bool vec = (a.V & 7) == 0;
  const long e0 = (long)c * kChunk1 + tid * 8;

  double x[2][8];
  load8(row, e0, a.V, vec, x[0]);
  load8(row, e0 + kThreads * 8, a.V, vec, x[1]);
  double mx = -INFINITY;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmax(mx, x[h][j]);
  mx = block_max_d(mx, shd);
  double s = 0.0;
  if (mx > -INFINITY) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) s += exp((x[h][j] - mx) / a.T);
  }
  s = block_sum_d(s, shd);
  if (tid == 0) {
    uint64_t* p = a.part1 + ((size_t)r * a.chunks1 + c) * 2;
    st_coherent(p, dbits(mx));
    st_coherent(p + 1, dbits(s));
  }
  // counter[1 + r]: chunks of row r; counter[0]: finished rows.
  if (!arrive_last(&a.counter[1 + r], (unsigned)a.chunks1)) return;

  const uint64_t* pr = a.part1 + (size_t)r * a.chunks1 * 2;
  double rmx = -INFINITY;
  for (int j = tid; j < a.chunks1; j += kThreads) rmx = fmax(rmx, bitsd(ld_coherent(&pr[2 * j])));
  rmx = block_max_d(rmx, shd);
  double rs = 0.0;
  for (int j = tid; j < a.chunks1; j += kThreads) {
    const double cm = bitsd(ld_coherent(&pr[2 * j]));
    const double cs = bitsd(ld_coherent(&pr[2 * j + 1]));
    if (cs > 0.0) rs += cs * exp((cm - rmx) / a.T);
  }
  rs = block_sum_d(rs, shd);
  if (tid == 0) {
    st_coherent(&a.rowstat[2 * r], dbits(rmx));
    st_coherent(&a.rowstat[2 * r + 1], dbits(rs));
  }
  if (!arrive_last(&a.counter[0], (unsigned)a.rows)) return;

  // Acceptance of draft i (thread i of wave 0): u[i] * q_i(x_i) < p_i(x_i).
  if (tid < kWave) {
    bool rejected = false;
    if (lane < a.M - 1) {
      const int xi = a.draft[lane];
      rejected = true;
      if (xi >= 0 && xi < a.V) {
        const double pm = bitsd(ld_coherent(&a.rowstat[2 * lane]));
        const double ps = bitsd(ld_coherent(&a.rowstat[2 * lane + 1]));
        const double p = exp((h2d(a.logits[(size_t)lane * a.V + xi]) - pm) / a.T) / ps;
        double q = 1.0;
        if (a.dlogits) {
          const int rq = a.M + lane;
          const double qm = bitsd(ld_coherent(&a.rowstat[2 * rq]));
          const double qs = bitsd(ld_coherent(&a.rowstat[2 * rq + 1]));
          q = exp((h2d(a.dlogits[(size_t)lane * a.V + xi]) - qm) / a.T) / qs;
        }
        rejected = !(a.u[lane] * q < p);
      }
    }
    const uint64_t mask = __ballot(rejected);
    if (lane == 0) {
      const int n = mask ? (int)__builtin_ctzll(mask) : a.M - 1;
      a.result[0] = n;
      a.sel[0] = n;
    }
  }
}

// ---- pass 2: the emitted token ---------------------------------------------------------
struct DrawRow {
  const uint16_t* p_row;
  const uint16_t* q_row;  // null: point mass at xq (none if xq is outside [0, V))
  double pm, ps, qm, qs;
  int xq;
  bool residual;
};

__device__ __forceinline__ DrawRow draw_row(const SampleArgs& a) {
  DrawRow d;
  const int n = a.sel[0];
  d.residual = n < a.M - 1;
  d.p_row = a.logits + (size_t)n * a.V;
  d.pm = bitsd(a.rowstat[2 * n]);
  d.ps = bitsd(a.rowstat[2 * n + 1]);
  d.q_row = nullptr;
  d.qm = d.qs = 0.0;
  d.xq = -1;
  if (d.residual) {
    d.xq = a.draft[n];
    if (a.dlogits) {
      d.q_row = a.dlogits + (size_t)n * a.V;
      d.qm = bitsd(a.rowstat[2 * (a.M + n)]);
      d.qs = bitsd(a.rowstat[2 * (a.M + n) + 1]);
    }
  }
  return d;
}

// Weights of the eight elements e .. e+7: p and (when residual) max(0, p - q); elements
// past V weigh 0.
__device__ __forceinline__ void weights8(const SampleArgs& a, const DrawRow& d, long e, bool vec,
                                         double (&p)[8], double (&w)[8]) {
  double x[8];
  load8(d.p_row, e, a.V, vec, x);
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = e + j < a.V ? exp((x[j] - d.pm) / a.T) / d.ps : 0.0;
  if (!d.residual) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = p[j];
    return;
  }
  double q[8];
  if (d.q_row) {
    load8(d.q_row, e, a.V, vec, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = e + j < a.V ? exp((x[j] - d.qm) / a.T) / d.qs : 0.0;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = e + j == d.xq ? 1.0 : 0.0;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = fmax(p[j] - q[j], 0.0);
}

__global__ __launch_bounds__(kThreads) void sample_draw_kernel(SampleArgs a) {
  const int c = blockIdx.x, tid = threadIdx.x;
  __shared__ double shd[kWaves];
  __shared__ int shi[kWaves];
  const bool vec = (a.V & 7) == 0;
  const DrawRow d = draw_row(a);

  double p[8], w[8];
  weights8(a, d, (long)c * kChunk2 + tid * 8, vec, p, w);
  double sw = 0.0, sp = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sw += w[j];
    sp += p[j];
  }
  sw = block_sum_d(sw, shd);
  sp = block_sum_d(sp, shd);
  if (tid == 0) {
    st_coherent(&a.part2[2 * c], dbits(sw));
    st_coherent(&a.part2[2 * c + 1], dbits(sp));
  }
  if (!arrive_last(&a.counter[kDrawCounter], (unsigned)a.chunks2)) return;

  // Chunk level: thread t owns chunks [t * span, (t + 1) * span).  Residual weights unless
  // they are all zero, then p.
  const int span = (a.chunks2 + kThreads - 1) / kThreads;
  const int c0 = tid * span, c1 = min(c0 + span, a.chunks2);
  double tw = 0.0, tp = 0.0;
  for (int j = c0; j < c1; ++j) {
    tw += bitsd(ld_coherent(&a.part2[2 * j]));
    tp += bitsd(ld_coherent(&a.part2[2 * j + 1]));
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
  // failing that, of the row.
  __shared__ int s_chunk;
  __shared__ double s_base;
  const int owner = block_first(incl > t, shi);
  const int who = owner >= 0 ? owner : block_last(mine > 0.0, shi);
  if (tid == 0) s_chunk = -1;
  __syncthreads();
  if (who >= 0 && tid == who) {
    double run = excl;
    int found = -1, last = -1;
    double found_base = 0.0, last_base = 0.0;
    for (int j = c0; j < c1; ++j) {
      const double v = bitsd(ld_coherent(&a.part2[2 * j + k]));
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
  __syncthreads();
  const int cs = s_chunk;
  if (cs < 0) {  // no positive weight anywhere (non-finite logits)
    if (tid == 0) a.result[1] = -1;
    return;
  }
  const bool exact = owner >= 0;  // otherwise take the chunk's last element of positive weight

  // Element level inside chunk cs: thread t owns elements cs * kChunk2 + 8t .. 8t+7.
  const long e = (long)cs * kChunk2 + tid * 8;
  weights8(a, d, e, vec, p, w);
  double ew[8];
  double own = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ew[j] = use_w ? w[j] : p[j];
    own += ew[j];
  }
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
    a.result[1] = pick >= 0 ? (int)(e + pick) : -1;
  }
  if (ewho < 0 && tid == 0) a.result[1] = -1;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

// Workspace after the counters: chunk statistics [rows][chunks1][2], row statistics
// [rows][2], the emitting row, chunk weights [chunks2][2]; each part 256-byte aligned.
// Sized for the drafter's rows present (rows = 2M - 1).
size_t sample_partial_bytes(int M, int V) {
  const size_t rows = 2 * (size_t)M - 1;
  const size_t c1 = ((size_t)V + kChunk1 - 1) / kChunk1, c2 = ((size_t)V + kChunk2 - 1) / kChunk2;
  return align256(rows * c1 * 16) + align256(rows * 16) + 256 + align256(c2 * 16);
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
  a.M = M;
  a.V = V;
  a.rows = M + (a.dlogits ? M - 1 : 0);
  a.chunks1 = (V + kChunk1 - 1) / kChunk1;
  a.chunks2 = (V + kChunk2 - 1) / kChunk2;
  a.result = result_out;
  a.counter = counters;
  const size_t rows_max = 2 * (size_t)M - 1;
  char* base = static_cast<char*>(partials);
  a.part1 = reinterpret_cast<uint64_t*>(base);
  base += align256(rows_max * a.chunks1 * 16);
  a.rowstat = reinterpret_cast<uint64_t*>(base);
  base += align256(rows_max * 16);
  a.sel = reinterpret_cast<int32_t*>(base);
  base += 256;
  a.part2 = reinterpret_cast<uint64_t*>(base);
  sample_stats_kernel<<<dim3(a.chunks1, a.rows), kThreads, 0, stream>>>(a);
  if (hipError_t e = hipGetLastError()) return e;
  sample_draw_kernel<<<a.chunks2, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace qv
