// Internal declarations shared by the HIP translation units of libqv.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qv.h"
#include "qv_test.h"

namespace qv {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- split-K exchange between workgroups, without cache-wide fences --------------------
// On gfx950 an agent-scope release/acquire fence writes back and invalidates the whole L2
// of the issuing XCD, which costs tens of microseconds when every workgroup of a split-K
// GEMM does it.  Instead, partial results are written with agent-scope atomic stores (they
// go to the device coherence point, not only to this XCD's L2) and read back with
// agent-scope atomic loads; each wave waits for its own stores to complete before the
// workgroup counts its arrival, so when the counter reaches the total every partial is
// visible to the workgroup that arrived last.
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_coherent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp16 bits of f32(v * s): the product rounded to fp32, then to fp16.  The empty asm pins
// the fp32 rounding: without it the compiler folds the product and the conversion into
// v_fma_mixlo_f16, which rounds once, so the same sum could give different bits in
// different kernels (one conversion fused, another not).
__device__ __forceinline__ uint16_t f16_of_product(float v, float s) {
  float t = v * s;
  asm("" : "+v"(t));
  return __builtin_bit_cast(uint16_t, (_Float16)t);
}

// Four consecutive fp32 values (16-byte aligned) moved with agent-scope visibility: loads as
// two 64-bit coherent atomics, stores as one 16-byte write-through store.
__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) | ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}
// The 16-byte store carries the same cache policy as an agent-scope atomic store (sc1:
// written through to the device coherence point) in one instruction.  It is a vector-memory
// store the compiler does not track; every reader is ordered behind it by arrive_last,
// whose s_waitcnt(0) waits for all of the wave's outstanding stores.  A store of more than
// 8 bytes still reads its data registers in the cycle after it issues, and a vector ALU
// write to them there would be stored instead; the compiler's hazard checks do not look
// inside inline assembly, so the s_nop provides the wait states.
__device__ __forceinline__ void st_coherent_f4(float* p, f32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ f32x4 ld_coherent_f4(const float* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  const uint64_t a = ld_coherent(q), b = ld_coherent(q + 1);
  return f32x4{__builtin_bit_cast(float, (uint32_t)a), __builtin_bit_cast(float, (uint32_t)(a >> 32)),
               __builtin_bit_cast(float, (uint32_t)b), __builtin_bit_cast(float, (uint32_t)(b >> 32))};
}

// Counts this workgroup's arrival at `counter` (after its coherent stores are complete) and
// returns true, uniformly across the workgroup, in the workgroup that arrives last of
// `total`.  That workgroup re-arms the counter to zero for the next call.
__device__ __forceinline__ bool arrive_last(unsigned* counter, unsigned total) {
  __shared__ int last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == total - 1;
    if (last) st_coherent(counter, 0u);
  }
  __syncthreads();
  return last != 0;
}

// Work split chosen by the host for one GEMM call.  `splits` workgroups share each output
// tile along K; with splits > 1 the workspace holds their partial sums and one arrival
// counter per output tile.
struct GemmPlan {
  int waves;        // waves per output tile (per workgroup unless nt > 1)
  int nt;           // output tiles per workgroup
  int tiles;        // output tiles (workgroups along N)
  int splits;       // workgroups along K per output tile
  int k_per_split;  // K elements per split (a multiple of the K step)
  int variant;      // kernel instantiation selector
  int ring;         // K-steps in flight per lane (W8A8 weight ring: 8 or 16)
  size_t partial_bytes;
  bool ok;          // false: the shape has no launchable plan (the call returns QV_ERR_SHAPE)
  bool reduce_launch;  // splits > 1: the partials are added by a second launch, not by the
                       // last workgroup of each tile block (no arrival counters then)
};

// Work-split overrides of one call (the QV_TUNE_* keys of qv_test.h).  The calls of qv.h pass
// kNoTuning, so their plans depend on the shape alone; only the qv_test_* entry points pass
// others.  A plain value read: no lock, no allocation, no process-wide state.
struct Tuning {
  int32_t v[QV_TUNE_COUNT];
  int operator()(int key) const { return v[key] > 0 ? v[key] : 0; }
};
extern const Tuning kNoTuning;

GemmPlan plan_w8a8(int M, int N, int K, const Tuning& t);
GemmPlan plan_w4a16(int M, int N, int K, bool vec_ok, const Tuning& t);
GemmPlan plan_w4a8(int M, int N, int K, const Tuning& t);
size_t verify_partial_bytes(int M, int V);
size_t sample_partial_bytes(int M, int V);

hipError_t launch_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                            int8_t* x_q, float* x_scale, hipStream_t stream, const Tuning& t);
hipError_t launch_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K,
                             int8_t* w_q, float* w_scale, hipStream_t stream, const Tuning& t);
hipError_t launch_prepare_w4(const uint16_t* w_bf16, int N, int K, uint32_t* qweight,
                             uint16_t* scales, uint8_t* zeros, hipStream_t stream);
hipError_t launch_w8a8(const GemmPlan& p, const int8_t* x_q, const float* x_scale, int M, int K,
                       const int8_t* w, const float* w_scale, int N, uint16_t* y,
                       int32_t* acc_out, unsigned* counters, void* partials, hipStream_t stream);
// y[m][n] = fp16(sum over s < splits of part[s][m][n]), times row_scale[m] if row_scale is
// not null, for an M x N output (N % 4 == 0), the splits added in order from +0: the split-K
// finish as a launch of its own, after a GEMM kernel that stored its fp32 partial sums with
// plain stores (the launch boundary orders them).
hipError_t launch_reduce_splits(const float* part, int splits, int M, int N,
                                const float* row_scale, uint16_t* y, hipStream_t stream);
hipError_t launch_w4a16(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream);
hipError_t launch_w4a8(const GemmPlan& p, const int8_t* xq, const float* sx, int M, int K,
                       const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros, int N,
                       uint16_t* y, unsigned* counters, void* partials, hipStream_t stream);
hipError_t launch_verify(const uint16_t* logits, int M, int V, const int32_t* draft,
                         int32_t* argmax_out, int32_t* n_accept_out, unsigned* counters,
                         void* partials, hipStream_t stream);
hipError_t launch_verify_tree(const uint16_t* logits, int M, int V, const int32_t* tokens,
                              const int32_t* parent, int32_t* argmax_out, int32_t* path_out,
                              int32_t* accept_out, unsigned* counters, void* partials,
                              hipStream_t stream);

hipError_t launch_verify_sample(const uint16_t* logits, int M, int V, const uint16_t* draft_logits,
                                const int32_t* draft, const double* uniforms, double temperature,
                                int32_t* result_out, unsigned* counters, void* partials,
                                hipStream_t stream);

}  // namespace qv
