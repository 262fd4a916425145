// C ABI of libqv.so: host-side argument checks, work-split planning and launches on the
// caller's stream.  Every check runs before any HIP call, so a rejected call has no effect
// on the device.
#include <math.h>
#include <string.h>

#include "qv_internal.h"

namespace qv {

const Tuning kNoTuning = {};

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_m(int M) { return M >= 1 && M <= QV_MAX_M; }

bool w8a8_shape_ok(int M, int N, int K) {
  return valid_m(M) && K >= 64 && K <= QV_W8A8_MAX_K && K % 64 == 0 && N >= 16 && N % 16 == 0;
}

bool w4a16_shape_ok(int M, int N, int K) {
  return valid_m(M) && K >= 128 && K <= QV_W4A16_MAX_K && K % 128 == 0 && N >= 16 &&
         N % 16 == 0 && (long long)N * (K / 8) < (1LL << 40);
}

bool verify_shape_ok(int M, int V) { return valid_m(M) && V >= 1 && V <= (1 << 30); }

size_t with_counters(size_t partial_bytes) {
  return partial_bytes ? QV_WORKSPACE_COUNTER_BYTES + partial_bytes : 0;
}

qv_status_t check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return QV_OK;
  if (ws == nullptr || have < need) return QV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QV_ERR_ALIGN;
  return QV_OK;
}

qv_status_t from_hip(hipError_t e) { return e == hipSuccess ? QV_OK : QV_ERR_HIP; }

Tuning tuning_from(const int32_t* tune) {
  Tuning t = kNoTuning;
  if (tune) memcpy(t.v, tune, sizeof(t.v));
  return t;
}

qv_status_t quant_act(const uint16_t* x, const float* inv_smooth, int M, int K, int8_t* x_q,
                      float* x_scale, void* stream, const Tuning& t) {
  if (!x || !x_q || !x_scale) return QV_ERR_NULL;
  if (!valid_m(M) || K < 8 || K % 8 != 0) return QV_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(x_q, 16) || !aligned(x_scale, 4) ||
      (inv_smooth && !aligned(inv_smooth, 4)))
    return QV_ERR_ALIGN;
  return from_hip(launch_quant_act(x, inv_smooth, M, K, x_q, x_scale, (hipStream_t)stream, t));
}

qv_status_t prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K, int8_t* w_q,
                       float* w_scale, void* stream, const Tuning& t) {
  if (!w_bf16 || !w_q || !w_scale) return QV_ERR_NULL;
  if (N < 1 || K < 8 || K % 8 != 0) return QV_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4) ||
      (inv_s && !aligned(inv_s, 4)))
    return QV_ERR_ALIGN;
  return from_hip(launch_prepare_w8(w_bf16, inv_s, N, K, w_q, w_scale, (hipStream_t)stream, t));
}

qv_status_t linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K, const int8_t* w,
                        const float* w_scale, int N, uint16_t* y, int32_t* acc_out,
                        void* workspace, size_t workspace_bytes, void* stream, const Tuning& t) {
  if (!x_q || !x_scale || !w || !w_scale || !y) return QV_ERR_NULL;
  if (!w8a8_shape_ok(M, N, K)) return QV_ERR_SHAPE;
  if (!aligned(x_q, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(x_scale, 4) ||
      !aligned(w_scale, 4) || (acc_out && !aligned(acc_out, 16)))
    return QV_ERR_ALIGN;
  const GemmPlan p = plan_w8a8(M, N, K, t);
  if (!p.ok) return QV_ERR_SHAPE;
  const size_t need = with_counters(p.partial_bytes);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = need ? static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES : nullptr;
  return from_hip(launch_w8a8(p, x_q, x_scale, M, K, w, w_scale, N, y, acc_out, counters,
                              partials, (hipStream_t)stream));
}

qv_status_t linear_w4a16(const uint16_t* x, int M, int K, const uint32_t* qweight,
                         const uint16_t* scales, const uint8_t* zeros, int N, int group_size,
                         uint16_t* y, void* workspace, size_t workspace_bytes, void* stream,
                         const Tuning& t) {
  if (!x || !qweight || !scales || !zeros || !y) return QV_ERR_NULL;
  if (group_size != QV_W4A16_GROUP || !w4a16_shape_ok(M, N, K)) return QV_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(qweight, 16) || !aligned(y, 16) || !aligned(scales, 2))
    return QV_ERR_ALIGN;
  // 8-group scale/zero vectors need 16-byte aligned scales and 8-byte aligned zeros.
  const GemmPlan p = plan_w4a16(M, N, K, aligned(scales, 16) && aligned(zeros, 8), t);
  if (!p.ok) return QV_ERR_SHAPE;
  const size_t need = with_counters(p.partial_bytes);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = need ? static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES : nullptr;
  return from_hip(launch_w4a16(p, x, M, K, qweight, scales, zeros, N, y, counters, partials,
                               (hipStream_t)stream));
}

qv_status_t linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                        const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                        int N, int group_size, uint16_t* y, void* workspace,
                        size_t workspace_bytes, void* stream, const Tuning& t) {
  if (!x_q || !x_scale || !qweight || !scales || !zeros || !y) return QV_ERR_NULL;
  if (!w4a16_shape_ok(M, N, K) || group_size != QV_W4A16_GROUP) return QV_ERR_SHAPE;
  if (!aligned(x_q, 16) || !aligned(x_scale, 4) || !aligned(qweight, 16) || !aligned(scales, 2) ||
      !aligned(y, 16))
    return QV_ERR_ALIGN;
  const GemmPlan p = plan_w4a8(M, N, K, t);
  if (!p.ok) return QV_ERR_SHAPE;
  const size_t need = with_counters(p.partial_bytes);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = need ? static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES : nullptr;
  return from_hip(launch_w4a8(p, x_q, x_scale, M, K, qweight, scales, zeros, N, y, counters,
                              partials, (hipStream_t)stream));
}

size_t workspace_bytes(int op, int M, int N, int K, const Tuning& t) {
  switch (op) {
    case QV_OP_W8A8: {
      if (!w8a8_shape_ok(M, N, K)) return 0;
      const GemmPlan p = plan_w8a8(M, N, K, t);
      return p.ok ? with_counters(p.partial_bytes) : 0;
    }
    case QV_OP_W4A16: {
      if (!w4a16_shape_ok(M, N, K)) return 0;
      // enough for either plan (the call picks one from the scale/zero alignment)
      const GemmPlan a = plan_w4a16(M, N, K, true, t), b = plan_w4a16(M, N, K, false, t);
      const size_t pa = a.ok ? a.partial_bytes : 0, pb = b.ok ? b.partial_bytes : 0;
      return with_counters(pa > pb ? pa : pb);
    }
    case QV_OP_W4A8: {
      if (!w4a16_shape_ok(M, N, K)) return 0;
      const GemmPlan p = plan_w4a8(M, N, K, t);
      return p.ok ? with_counters(p.partial_bytes) : 0;
    }
    case QV_OP_VERIFY:
      return verify_shape_ok(M, N) ? QV_WORKSPACE_COUNTER_BYTES + verify_partial_bytes(M, N) : 0;
    case QV_OP_SAMPLE:
      return verify_shape_ok(M, N) ? QV_WORKSPACE_COUNTER_BYTES + sample_partial_bytes(M, N) : 0;
    default:
      return 0;
  }
}

}  // namespace
}  // namespace qv

using namespace qv;

extern "C" {

qv_status_t qv_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K, int8_t* x_q,
                         float* x_scale, void* stream) {
  return quant_act(x, inv_smooth, M, K, x_q, x_scale, stream, kNoTuning);
}

qv_status_t qv_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K, int8_t* w_q,
                          float* w_scale, void* stream) {
  return prepare_w8(w_bf16, inv_s, N, K, w_q, w_scale, stream, kNoTuning);
}

qv_status_t qv_prepare_w4(const uint16_t* w_bf16, int N, int K, int group_size, uint32_t* qweight,
                          uint16_t* scales, uint8_t* zeros, void* stream) {
  if (!w_bf16 || !qweight || !scales || !zeros) return QV_ERR_NULL;
  if (N < 1 || K < QV_W4A16_GROUP || K % QV_W4A16_GROUP != 0 || group_size != QV_W4A16_GROUP ||
      (long long)N * (K / QV_W4A16_GROUP) > (1LL << 31) * 16 * 4 - 64)
    return QV_ERR_SHAPE;
  if (!aligned(w_bf16, 16) || !aligned(qweight, 4) || !aligned(scales, 2)) return QV_ERR_ALIGN;
  return from_hip(launch_prepare_w4(w_bf16, N, K, qweight, scales, zeros, (hipStream_t)stream));
}

qv_status_t qv_linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K, const int8_t* w,
                           const float* w_scale, int N, uint16_t* y, int32_t* acc_out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return linear_w8a8(x_q, x_scale, M, K, w, w_scale, N, y, acc_out, workspace, workspace_bytes,
                     stream, kNoTuning);
}

qv_status_t qv_linear_w4a16(const uint16_t* x, int M, int K, const uint32_t* qweight,
                            const uint16_t* scales, const uint8_t* zeros, int N, int group_size,
                            uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  return linear_w4a16(x, M, K, qweight, scales, zeros, N, group_size, y, workspace,
                      workspace_bytes, stream, kNoTuning);
}

qv_status_t qv_linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                           const uint32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                           int N, int group_size, uint16_t* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return linear_w4a8(x_q, x_scale, M, K, qweight, scales, zeros, N, group_size, y, workspace,
                     workspace_bytes, stream, kNoTuning);
}

qv_status_t qv_verify_greedy(const uint16_t* logits, int M, int V, const int32_t* draft,
                             int32_t* argmax_out, int32_t* n_accept_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!logits || !argmax_out || !n_accept_out || (M > 1 && !draft)) return QV_ERR_NULL;
  if (!verify_shape_ok(M, V)) return QV_ERR_SHAPE;
  if (!aligned(logits, 16) || !aligned(argmax_out, 4) || !aligned(n_accept_out, 4) ||
      (draft && !aligned(draft, 4)))
    return QV_ERR_ALIGN;
  const size_t need = QV_WORKSPACE_COUNTER_BYTES + verify_partial_bytes(M, V);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES;
  return from_hip(launch_verify(logits, M, V, draft, argmax_out, n_accept_out, counters, partials,
                                (hipStream_t)stream));
}

qv_status_t qv_verify_tree(const uint16_t* logits, int M, int V, const int32_t* tokens,
                           const int32_t* parent, int32_t* argmax_out, int32_t* path_out,
                           int32_t* accept_out, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!logits || !tokens || !parent || !argmax_out || !path_out || !accept_out)
    return QV_ERR_NULL;
  if (!verify_shape_ok(M, V)) return QV_ERR_SHAPE;
  if (!aligned(logits, 16) || !aligned(tokens, 4) || !aligned(parent, 4) ||
      !aligned(argmax_out, 4) || !aligned(path_out, 4) || !aligned(accept_out, 4))
    return QV_ERR_ALIGN;
  const size_t need = QV_WORKSPACE_COUNTER_BYTES + verify_partial_bytes(M, V);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES;
  return from_hip(launch_verify_tree(logits, M, V, tokens, parent, argmax_out, path_out,
                                     accept_out, counters, partials, (hipStream_t)stream));
}

qv_status_t qv_verify_sample(const uint16_t* logits, int M, int V, const uint16_t* draft_logits,
                             const int32_t* draft, const double* uniforms, double temperature,
                             int32_t* result_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (!logits || !uniforms || !result_out || (M > 1 && !draft)) return QV_ERR_NULL;
  if (!verify_shape_ok(M, V) || !(temperature > 0.0) || !isfinite(temperature))
    return QV_ERR_SHAPE;
  if (M == 1) draft_logits = nullptr;
  if (!aligned(logits, 16) || (draft_logits && !aligned(draft_logits, 16)) ||
      (draft && !aligned(draft, 4)) || !aligned(uniforms, 8) || !aligned(result_out, 4))
    return QV_ERR_ALIGN;
  const size_t need = QV_WORKSPACE_COUNTER_BYTES + sample_partial_bytes(M, V);
  if (qv_status_t s = check_workspace(workspace, workspace_bytes, need)) return s;
  unsigned* counters = static_cast<unsigned*>(workspace);
  void* partials = static_cast<char*>(workspace) + QV_WORKSPACE_COUNTER_BYTES;
  return from_hip(launch_verify_sample(logits, M, V, draft_logits, M > 1 ? draft : nullptr,
                                       uniforms, temperature, result_out, counters, partials,
                                       (hipStream_t)stream));
}

size_t qv_workspace_bytes(int op, int M, int N, int K) {
  return workspace_bytes(op, M, N, K, kNoTuning);
}

const char* qv_status_str(qv_status_t s) {
  switch (s) {
    case QV_OK: return "ok";
    case QV_ERR_NULL: return "a required pointer is NULL";
    case QV_ERR_SHAPE: return "a size is outside the supported shape rules";
    case QV_ERR_ALIGN: return "a pointer is not aligned as required";
    case QV_ERR_WORKSPACE: return "workspace missing or smaller than qv_workspace_bytes()";
    case QV_ERR_HIP: return "the HIP runtime rejected a launch";
    case QV_ERR_SCRATCH: return "the shape needs more than the static scratch of the no-allocation call";
    default: return "unknown status";
  }
}

// ---- qv_test.h: the same calls with work-split overrides -------------------------------

qv_status_t qv_test_quant_act(const uint16_t* x, const float* inv_smooth, int M, int K,
                              int8_t* x_q, float* x_scale, void* stream, const int32_t* tune) {
  return quant_act(x, inv_smooth, M, K, x_q, x_scale, stream, tuning_from(tune));
}

qv_status_t qv_test_prepare_w8(const uint16_t* w_bf16, const float* inv_s, int N, int K,
                               int8_t* w_q, float* w_scale, void* stream, const int32_t* tune) {
  return prepare_w8(w_bf16, inv_s, N, K, w_q, w_scale, stream, tuning_from(tune));
}

qv_status_t qv_test_linear_w8a8(const int8_t* x_q, const float* x_scale, int M, int K,
                                const int8_t* w, const float* w_scale, int N, uint16_t* y,
                                int32_t* acc_out, void* workspace, size_t workspace_bytes,
                                void* stream, const int32_t* tune) {
  return linear_w8a8(x_q, x_scale, M, K, w, w_scale, N, y, acc_out, workspace, workspace_bytes,
                     stream, tuning_from(tune));
}

qv_status_t qv_test_linear_w4a16(const uint16_t* x, int M, int K, const uint32_t* qweight,
                                 const uint16_t* scales, const uint8_t* zeros, int N,
                                 int group_size, uint16_t* y, void* workspace,
                                 size_t workspace_bytes, void* stream, const int32_t* tune) {
  return linear_w4a16(x, M, K, qweight, scales, zeros, N, group_size, y, workspace,
                      workspace_bytes, stream, tuning_from(tune));
}

qv_status_t qv_test_linear_w4a8(const int8_t* x_q, const float* x_scale, int M, int K,
                                const uint32_t* qweight, const uint16_t* scales,
                                const uint8_t* zeros, int N, int group_size, uint16_t* y,
                                void* workspace, size_t workspace_bytes, void* stream,
                                const int32_t* tune) {
  return linear_w4a8(x_q, x_scale, M, K, qweight, scales, zeros, N, group_size, y, workspace,
                     workspace_bytes, stream, tuning_from(tune));
}

size_t qv_test_workspace_bytes(int op, int M, int N, int K, const int32_t* tune) {
  return workspace_bytes(op, M, N, K, tuning_from(tune));
}

int qv_version(void) { return 100; }

}  // extern "C"
