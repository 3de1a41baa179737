// HBM read probes for the bench: what the chip delivers for
//   (a) one long contiguous read, and
//   (b) random pages of 8 KiB (bf16 keys) or 4 KiB (fp8 codes) read the way
//       the score kernel reads its keys: a fixed grid of one-wave workgroups,
//       each over an equal contiguous range of a page-id list, 1 KiB wave
//       loads (non-temporal), two pages in flight per wave, and nothing else
//       (no page-table walk, no scales, no compute, no stores but one word
//       per lane at the end).
// They measure the ceiling of the access pattern, not a step of the method.
// Each wave folds what it read into one word per lane, so no load is dead.
// Every access goes through a buffer resource sized to its buffer, so nothing
// outside the buffers is touched whatever the arguments.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}
__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// (a) contiguous read: 16-byte chunk i of the buffer is read by thread
// i % n_threads, kU chunks in flight per thread, with cache policy kPolicy.
template <int kU, int kPolicy>
__global__ __launch_bounds__(256) void stream_read(const void* src, uint32_t chunks, uint32_t* out) {
  const rsrc_t r = make_rsrc(src, chunks * 16u);
  const uint32_t n_threads = gridDim.x * blockDim.x;
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  uint32_t i = t;
  for (; i + (kU - 1) * n_threads < chunks; i += kU * n_threads) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (i + u * n_threads) * 16, 0, kPolicy);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= fold(v[u]);
  }
  for (; i < chunks; i += n_threads) acc ^= fold(__builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, kPolicy));
  const rsrc_t o = make_rsrc(out, n_threads * 4u);
  __builtin_amdgcn_raw_buffer_store_b32(acc, o, t * 4, 0, 0);
}

// (b) random pages: workgroup g reads pages ids[g * per .. min(n_ids, (g + 1) * per)).
template <int kPageBytes>
__global__ __launch_bounds__(64) void page_read(const void* pool, uint32_t pool_bytes, const int32_t* ids,
                                                int32_t n_ids, uint32_t* out) {
  constexpr int kLoads = kPageBytes / 1024;
  const int lane = threadIdx.x;
  const int per = (n_ids + (int)gridDim.x - 1) / (int)gridDim.x;
  const int s = min(n_ids, (int)blockIdx.x * per), e = min(n_ids, s + per);
  const rsrc_t ir = make_rsrc(ids, (uint32_t)n_ids * 4u);
  uint32_t acc = 0;
  u32x4 a[kLoads], b[kLoads];
  int id_block = -1;
  int my_id = 0;  // lane l: the id of item id_block * 64 + l
  auto issue = [&](int item, u32x4 (&dst)[kLoads]) {
    int page = 0;
    const bool in = item < e;
    if (in) {
      if ((item >> 6) != id_block) {
        id_block = item >> 6;
        my_id = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (id_block * 64 + lane) * 4, 0, 0);
      }
      page = __builtin_amdgcn_readlane(my_id, item & 63);
    }
    const uint64_t off = (uint64_t)(uint32_t)page * kPageBytes;
    const bool ok = in && page >= 0 && off + kPageBytes <= pool_bytes;
    const rsrc_t pr = make_rsrc(static_cast<const char*>(pool) + (ok ? off : 0), ok ? kPageBytes : 0u);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b128(pr, (i * 64 + lane) * 16, 0, kNonTemporal);
  };
  if (s < e) {
    issue(s, a);
    for (int it = s; it < e; it += 2) {
      issue(it + 1, b);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) acc ^= fold(a[i]);
      if (it + 1 >= e) break;
      issue(it + 2, a);
#pragma unroll
      for (int i = 0; i < kLoads; ++i) acc ^= fold(b[i]);
    }
  }
  const rsrc_t o = make_rsrc(out, gridDim.x * 256u);
  __builtin_amdgcn_raw_buffer_store_b32(acc, o, (blockIdx.x * 64 + lane) * 4, 0, 0);
}

}  // namespace

// src: `bytes` of device memory (a multiple of 16, below 4 GiB); out: one
// uint32 per thread of the grid (grid * 256 words); variant 0..3: 4 or 8
// chunks in flight per thread, streaming or default cache policy. Returns a
// hipError_t.
extern "C" int dsa_probe_stream_read(const void* src, uint64_t bytes, uint32_t* out, int grid, int variant,
                                     hipStream_t stream) {
  if (!src || !out || grid < 1 || bytes % 16 != 0 || bytes == 0 || bytes >= (uint64_t(1) << 32))
    return (int)hipErrorInvalidValue;
  const uint32_t chunks = (uint32_t)(bytes / 16);
  switch (variant) {
    case 0: hipLaunchKernelGGL((stream_read<4, kNonTemporal>), dim3(grid), dim3(256), 0, stream, src, chunks, out); break;
    case 1: hipLaunchKernelGGL((stream_read<8, kNonTemporal>), dim3(grid), dim3(256), 0, stream, src, chunks, out); break;
    case 2: hipLaunchKernelGGL((stream_read<4, 0>), dim3(grid), dim3(256), 0, stream, src, chunks, out); break;
    case 3: hipLaunchKernelGGL((stream_read<8, 0>), dim3(grid), dim3(256), 0, stream, src, chunks, out); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// pool: pool_bytes of pages of page_bytes (8192 or 4096; below 4 GiB in
// all); ids: n_ids page ids (an id outside the pool reads nothing); out:
// grid * 64 words. Returns a hipError_t.
extern "C" int dsa_probe_page_read(const void* pool, uint64_t pool_bytes, const int32_t* ids, int n_ids, uint32_t* out,
                                   int grid, int page_bytes, hipStream_t stream) {
  if (!pool || !ids || !out || grid < 1 || n_ids < 1 || pool_bytes >= (uint64_t(1) << 32))
    return (int)hipErrorInvalidValue;
  if (page_bytes == 8192)
    hipLaunchKernelGGL(page_read<8192>, dim3(grid), dim3(64), 0, stream, pool, (uint32_t)pool_bytes, ids, n_ids, out);
  else if (page_bytes == 4096)
    hipLaunchKernelGGL(page_read<4096>, dim3(grid), dim3(64), 0, stream, pool, (uint32_t)pool_bytes, ids, n_ids, out);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
