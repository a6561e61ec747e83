// qsa_forward_noalloc: qsa_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  The workspace qsa_forward takes from its caller (the
// compacted lists and counts, then the key-range split's range starts and
// partial results) lives instead in `scratch`, a file-scope device array of
// QSA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends.  The kernels are qsa_forward's, given the array's device
// address as their workspace pointer.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device, with that device current,
// with hipGetSymbolAddress, and only that address is ever handed to a
// kernel.  Nothing in the scratch needs to start at zero (every kernel writes
// what it later reads); calls that overlap on one GPU share the array and
// race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qsa.h"
#include "qsa_internal.h"

static __device__ __align__(256) uint8_t scratch[QSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array; the stream must
// belong to that device.
int scratch_for_stream(size_t need, void* stream, void** workspace, size_t* workspace_bytes) {
  if (need > QSA_NOALLOC_SCRATCH_BYTES) return QSA_ERR_SCRATCH_LIMIT;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QSA_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t stream_dev = -1;
    if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &stream_dev) != hipSuccess || stream_dev != dev)
      return QSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *workspace = g_scratch_ptr[dev];
  *workspace_bytes = QSA_NOALLOC_SCRATCH_BYTES;
  return QSA_OK;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int qsa_forward_noalloc(
    const void* q, const int64_t q_strides[4], const void* k, const int64_t k_strides[4], const void* v,
    const int64_t v_strides[4], const void* routes, int routes_dtype, const int64_t route_strides[3], int64_t B,
    int64_t S_q, int64_t S_kv, int64_t Hq, int64_t Hkv, int64_t D, int64_t K, float scale, void* out,
    void* stream) {
  return qsa::forward_entry(q, q_strides, k, k_strides, v, v_strides, routes, routes_dtype, route_strides, B, S_q,
                            S_kv, Hq, Hkv, D, K, scale, out, nullptr, 0, scratch_for_stream, stream);
}
