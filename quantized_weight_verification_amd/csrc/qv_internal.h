// Internal declarations shared by the HIP translation units of libqv.so (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qv.h"

namespace qv {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Work split chosen by the host for one GEMM call.  `splits` workgroups share each output
// tile along K; with splits > 1 the workspace holds their partial sums and one arrival
// counter per output tile.
struct GemmPlan {
  int waves;        // waves per workgroup
  int tiles;        // output tiles (workgroups along N)
  int splits;       // workgroups along K per output tile
  int k_per_split;  // K elements per split (a multiple of the K step)
  int variant;      // kernel instantiation selector
  size_t partial_bytes;
};

GemmPlan plan_w8a8(int M, int N, int K);
GemmPlan plan_w4a16(int M, int N, int K);
size_t verify_partial_bytes(int M, int V);

hipError_t launch_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                            int8_t* x_q, float* x_scale, hipStream_t stream);
hipError_t launch_w8a8(const GemmPlan& p, const int8_t* x_q, const float* x_scale, int M, int K,
                       const int8_t* w, const float* w_scale, int N, uint16_t* y,
                       int32_t* acc_out, unsigned* counters, void* partials, hipStream_t stream);
hipError_t launch_w4a16(const GemmPlan& p, const uint16_t* x, int M, int K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int N, uint16_t* y,
                        unsigned* counters, void* partials, hipStream_t stream);
hipError_t launch_verify(const uint16_t* logits, int M, int V, const int32_t* draft,
                         int32_t* argmax_out, int32_t* n_accept_out, unsigned* counters,
                         void* partials, hipStream_t stream);

// Tuning overrides read once from the environment (QV_W8A8_SPLITS, QV_W8A8_WAVES,
// QV_W4A16_SPLITS, ...); 0 = use the built-in plan.
int tune_env(const char* name);

}  // namespace qv
