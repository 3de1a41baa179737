// Top-k for callers that cannot allocate device memory: code under hipGraph
// capture, tight serving loops, harnesses that forbid hipMalloc. The same
// kernels as dsa_indexer_topk, with their workspace (needed only for a row
// width above 32768 positions) in a fixed device array instead of a caller
// buffer.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy, at its own address, from module load until the process
// ends. In host code its name is only a stand-in, so the device address is
// resolved once per device (hipGetSymbolAddress, with that device current) on
// the first call there, kept, and passed to the kernels like the caller's
// workspace. The top-k writes every workspace word it reads within one call,
// so the array needs no clearing; calls that overlap on one GPU (other
// streams, other threads) share it and race.
#include <mutex>

#include "dsa_indexer.h"

#include "common.h"

static __device__ __align__(256) unsigned char scratch[DSA_INDEXER_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device `stream` enqueues on (the current device for the null stream).
hipError_t stream_device(hipStream_t stream, int* dev) {
  if (stream != nullptr) return hipStreamGetDevice(stream, dev);
  return hipGetDevice(dev);
}

// Device address of device dev's copy of the array, resolved on first use.
hipError_t scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int dsa_indexer_topk_noalloc(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                                        int32_t k, int32_t* out_idx, float* out_vals, hipStream_t stream) {
  if (!logits || !seq_lens || !out_idx) return DSA_ERR_NULL;
  if (batch < 1 || batch > 65535 || max_c4 < 1 || max_c4 > dsa::kMaxRowPositions) return DSA_ERR_SHAPE;
  if (k < 1 || k > max_c4) return DSA_ERR_K;
  if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (reinterpret_cast<uintptr_t>(out_idx) & 3u) || (reinterpret_cast<uintptr_t>(out_vals) & 3u))
    return DSA_ERR_ALIGN;
  const size_t need = dsa::topk_workspace_words(batch, max_c4) * sizeof(uint32_t);
  if (need > (size_t)DSA_INDEXER_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    int dev = 0;
    hipError_t e = stream_device(stream, &dev);
    if (e == hipSuccess) e = scratch_on(dev, &ws);
    if (e != hipSuccess) return dsa::record_hip_error(e);
  }
  return dsa::record_hip_error(
      dsa::launch_topk(logits, seq_lens, batch, max_c4, k, out_idx, out_vals, ws, nullptr, stream));
}
