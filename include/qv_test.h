/*
 * qv_test.h -- work-split overrides for testing and measurement (libqv.so).
 *
 * Callers: the parity tests that run every kernel configuration of a call, and launch-shape
 * measurements.  A production caller needs none of this: the calls of qv.h always run the
 * library's built-in plan, hold no state between calls and read no environment, so one
 * call gives the same bits in every process.
 *
 * Each qv_test_* call takes the arguments of its qv.h namesake followed by `tune`, an array
 * of QV_TUNE_COUNT int32 entries indexed by the QV_TUNE_* keys below (0 = the built-in choice
 * for that key), or NULL (the built-in plan: then the call is exactly its qv.h namesake).  A
 * value the kernel family has no instance for is rounded to the nearest one it has, or
 * ignored; the argument checks and error codes are those of qv.h.  Overrides change only
 * the launch shape: integer results (W8A8 accumulators, the int8 codes of quant_act and
 * qv_prepare_w8) are identical under every override, and fp32 summation order (the fp16
 * outputs of qv_linear_w4a16 and qv_linear_w4a8) may differ, within the bars stated in qv.h.
 * The workspace of a tuned call is sized by qv_test_workspace_bytes with the same `tune`.
 */
#ifndef QV_TEST_H
#define QV_TEST_H

#include "qv.h"

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QV_TUNE_W8A8_WAVES = 0,   /* waves per 16-channel tile: 2 (LDS-staged only), 4, 8, 16 */
  QV_TUNE_W8A8_SPLITS,      /* workgroups along K per tile */
  QV_TUNE_W8A8_RING,        /* 1 = LDS-staged activations with a weight ring, 2 = direct */
  QV_TUNE_W8A8_NT,          /* 16-channel tiles per LDS-staged workgroup: 1, 2, 4 */
  QV_TUNE_W8A8_RINGP,       /* K-steps in flight per lane in the ring: 8, 12, 16 */
  QV_TUNE_W4A16_CFG,        /* W4A16 kernel configuration index (see w4a16.hip) */
  QV_TUNE_W4A16_SPLITS,     /* workgroups along K per tile block */
  QV_TUNE_W4A8_NT,          /* tiles per workgroup: 1, 2, 4; 8, 10, 14, 16 for the chunked kernel */
  QV_TUNE_W4A8_WAVES,       /* waves per tile */
  QV_TUNE_W4A8_SPLITS,      /* workgroups along K */
  QV_TUNE_W4A8_LDS_KB,      /* LDS budget of the staged slice, KiB */
  QV_TUNE_W4A8_CG,          /* groups per chunk of the chunked kernel: 4, 8 */
  QV_TUNE_W4A8_STAGED,      /* 1 = the staged-slice kernel also at M > 16 */
  QV_TUNE_QUANT_SEGS,       /* workgroups per quantised row in qv_quant_act */
  QV_TUNE_PREP_W8_THREADS,  /* workgroup size of qv_prepare_w8: 128, 256, 512 */
  QV_TUNE_W4A16_REDUCE,     /* W4A16 split-K finish: 1 = last workgroup per tile, 2 = own launch */
  QV_TUNE_W4A8_REDUCE,      /* W4A8 (M > 16) split-K finish: 1 = last workgroup, 2 = own launch */
  QV_TUNE_COUNT
};

qv_status_t qv_test_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                              int8_t* x_q, float* x_scale, void* stream, const int32_t* tune);
qv_status_t qv_test_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K,
                               int8_t* w_q, float* w_scale, void* stream, const int32_t* tune);
qv_status_t qv_test_linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K,
                                const int8_t* w, const float* w_scale, int N, uint16_t* y,
                                int32_t* acc_out, void* workspace, size_t workspace_bytes,
                                void* stream, const int32_t* tune);
qv_status_t qv_test_linear_w4a16(const uint16_t* x, int M, int K, const uint32_t* qweight,
                                 const uint16_t* scales, const uint8_t* zeros, int N,
                                 int group_size, uint16_t* y, void* workspace,
                                 size_t workspace_bytes, void* stream, const int32_t* tune);
qv_status_t qv_test_linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                                const uint32_t* qweight, const uint16_t* scales,
                                const uint8_t* zeros, int N, int group_size, uint16_t* y,
                                void* workspace, size_t workspace_bytes, void* stream,
                                const int32_t* tune);
size_t qv_test_workspace_bytes(int op, int M, int N, int K, const int32_t* tune);

/*
 * Read-only bandwidth probe: the practical ceiling of a kernel that only streams memory, the
 * yardstick beside the published HBM peak for the weight-streaming GEMMs.  Reads `bytes` at
 * `src` (device memory, 16-byte aligned) once and writes, per workgroup of 256 threads, the XOR
 * of the 16-byte vectors it read to sink[16 b .. 16 b + 15] (b < blocks; sink is device memory,
 * 16-byte aligned, caller-owned, 16 * blocks bytes).  The XOR over all `blocks` entries equals
 * the XOR of every 16-byte vector of the buffer, for either pattern.
 *   pattern QV_READ_LINEAR: the buffer as one run of 16-byte vectors, grid-strided; `bytes` a
 *     multiple of 16; row_bytes ignored.
 *   pattern QV_READ_TILES: the layout of a weight matrix read by the GEMM kernels: rows of
 *     row_bytes (a positive multiple of 64), one wave per tile of 16 consecutive rows, each
 *     load instruction 64 bytes from each of the 16 rows, walking the rows from start to end;
 *     `bytes` a multiple of 16 * row_bytes.
 * nontemporal != 0 marks the loads non-temporal (streaming) for the caches.  blocks: 1 ..
 * QV_READ_MAX_BLOCKS.  Asynchronous on `stream`.  QV_ERR_NULL, QV_ERR_SHAPE, QV_ERR_ALIGN for
 * bad arguments (checked before anything is launched), QV_ERR_HIP if the launch fails.
 */
enum { QV_READ_LINEAR = 0, QV_READ_TILES = 1 };
#define QV_READ_MAX_BLOCKS 65536
qv_status_t qv_test_read_stream(const void* src, size_t bytes, int pattern, int row_bytes,
                                int nontemporal, int blocks, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QV_TEST_H */
