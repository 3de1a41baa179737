// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kHeads = 32;            // indexer heads
constexpr int kDim = 64;              // head dimension
constexpr int kPage = 64;             // c4 positions per page
constexpr int kRowBytes = kDim * 2;   // one bf16 key: 128 B
constexpr int kPageBytes = kPage * kRowBytes;  // 8 KiB
constexpr int kPageChunks = kPageBytes / 16;   // 512 chunks of 16 B

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Device memory is reached through raw buffer resources: a wave-uniform base
// and byte range in SGPRs plus a 32-bit per-lane byte offset. No per-lane
// 64-bit address is ever formed, and the hardware drops (or reads as 0) any
// access at or past the resource's range instead of touching other memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;  // dword 3 of a raw CDNA buffer descriptor
constexpr int kNonTemporal = 2;              // cache policy: streaming, read once
// Cache policy of a store that the next kernel reads (sc1): written through
// the XCD's L2, so that the writeback of dirty lines at the end of the kernel
// has little left to do and the next kernel starts earlier.
constexpr int kWriteThrough = 16;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRawBufferFlags);
}

// Monotone map float -> uint32 used by the top-k: a > b as floats (with -0 ==
// +0) iff key(a) > key(b). Non-negative floats get the sign bit set, negative
// ones are complemented; NaN maps to 1, below the key of every number (-inf
// maps to 0x007FFFFF). Key 0 marks a slot past a row's length, so a key is
// valid iff it is >= 1.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);  // -0 + 0 = +0
  const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return (x != x) ? 1u : key;
}

// Histogram of the first digit of the keys (their top kHistBits bits), per
// request: what the score kernel can count as it writes the logits, so that
// the top-k needs neither a sampled cut nor its first radix pass.
constexpr int kHistBits = 11;
constexpr int kHistBins = 1 << kHistBits;
constexpr int kHistShift = 32 - kHistBits;

// Largest row width (positions) either kernel accepts: keeps every row's
// byte range inside one 32-bit buffer range.
constexpr int32_t kMaxRowPositions = 1 << 28;

// DSA_OK for hipSuccess; otherwise keeps e for dsa_indexer_last_hip_error()
// on this thread and returns DSA_ERR_HIP.
int record_hip_error(hipError_t e);

// Enqueue the score kernel (with row_hwm, the incremental -inf tail: one mark
// per request, the longest of its tokens' lengths).
// hist: nullptr, or uint32 [B][kHistBins] to which the kernel adds, for every
// valid position of request b, one count in bin order_key(score) >> kHistShift
// (tokens == 1 only).
// k_scale == nullptr: bfloat16 keys; otherwise e4m3fn keys with these per-key
// scales (tokens == 1). tokens (1..4) query tokens per request: q [B][tokens][32][64],
// w [B][tokens][32], seq_lens [B][tokens], logits [B][tokens][width].
constexpr int32_t kMaxTokens = 4;
hipError_t launch_score(const void* q, const float* w, const void* k_pool, const float* k_scale,
                        int64_t num_pages, const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                        int32_t tokens, int32_t max_pages, float* logits, int32_t* row_hwm, uint32_t* hist,
                        hipStream_t stream);

// 32-bit words of top-k workspace for these sizes.
size_t topk_workspace_words(int32_t batch, int32_t max_c4);

// Enqueue the top-k kernels (workspace: topk_workspace_words words, any
// contents). hist: nullptr, or the score kernel's histograms of these logits,
// which then replace the sampled cut and the first radix pass; the row kernel
// sets every bin back to zero.
hipError_t launch_topk(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                       int32_t k, int32_t* out_idx, float* out_vals, void* workspace, uint32_t* hist,
                       hipStream_t stream);

// Sparse attention over the selected positions: 32 heads, 576-dim latents
// (the first 512 dims are the value), at most kMaxAttK list entries per request.
constexpr int32_t kMaxAttK = 2048;
constexpr int32_t kMaxAttChunk = 1024;  // list entries one workgroup handles at most
constexpr int kAttTargetGroups = 256;  // workgroups the split plan aims for (one per CU)

// Splits of each request's list (nsplit) and list entries per split (chunk).
void att_plan(int32_t batch, int32_t k, int32_t* nsplit, int32_t* chunk);

// Bytes of attention workspace for these sizes (0 when one split suffices).
size_t att_workspace_bytes(int32_t batch, int32_t k);

// Enqueue the attention kernel (and, with more than one split, the merge).
hipError_t launch_attention(const void* q, const void* kv, int64_t num_pages, const int32_t* page_table,
                            int32_t batch, int32_t max_pages, const int32_t* idx, int32_t k, float scale,
                            float* out, float* lse, void* workspace, hipStream_t stream);

}  // namespace dsa
