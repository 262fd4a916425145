// Greedy verification without a caller workspace: the arrival counters and chunk keys of
// verify_kernel live in a file-scope device array, one copy per GPU, so the call allocates
// nothing (for callers under HIP graph capture, in tight serving loops, or in harnesses that
// forbid allocation).
//
// Host code never uses the array's name as a device address (on the host it is only a stand-in
// for the symbol): the first call on each device resolves the array's address on that device
// with hipGetSymbolAddress and keeps it; every launch then gets that pointer.
#include <atomic>
#include <mutex>

#include "qv_internal.h"

namespace qv {
namespace {

// [0, kCounterBytes): arrival counters (verify uses M + 1 <= 65 of them); the rest: the chunk
// keys and row results of verify_kernel.
constexpr size_t kCounterBytes = 1024;
static __device__ __align__(256) unsigned char scratch[QV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_ptr[kMaxDevices];
std::mutex g_init;

__global__ void clear_words(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// The device address of `scratch` on the current device, resolved (and its counters cleared,
// in order on `stream`) on the device's first call.  nullptr if HIP refuses.
void* device_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_init);
  p = g_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  // Counters must start at zero; every verify call leaves them zero again.  A kernel, not a
  // memset, so that a first call under graph capture records no memset node.
  clear_words<<<1, 256, 0, stream>>>(static_cast<unsigned*>(q), (int)(kCounterBytes / 4));
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace
}  // namespace qv

using namespace qv;

extern "C" qv_status_t qv_verify_greedy_noalloc(const uint16_t* logits, int M, int V,
                                                const int32_t* draft, int32_t* argmax_out,
                                                int32_t* n_accept_out, void* stream) {
  if (!logits || !argmax_out || !n_accept_out || (M > 1 && !draft)) return QV_ERR_NULL;
  if (M < 1 || M > QV_MAX_M || V < 1 || V > (1 << 30)) return QV_ERR_SHAPE;
  if (kCounterBytes + verify_partial_bytes(M, V) > QV_NOALLOC_SCRATCH_BYTES) return QV_ERR_SCRATCH;
  if (((uintptr_t)logits % 16) != 0 || ((uintptr_t)argmax_out % 4) != 0 ||
      ((uintptr_t)n_accept_out % 4) != 0 || (draft && ((uintptr_t)draft % 4) != 0))
    return QV_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* base = static_cast<unsigned char*>(device_scratch(s));
  if (!base) return QV_ERR_HIP;
  const hipError_t e = launch_verify(logits, M, V, draft, argmax_out, n_accept_out,
                                     reinterpret_cast<unsigned*>(base), base + kCounterBytes, s);
  return e == hipSuccess ? QV_OK : QV_ERR_HIP;
}
