// Top-k kernel of the DSA indexer decode step on gfx950.
//
// What it computes (page "The O(Actual) Indexer", section "The Benchmark
// Results": the top-k that consumes the indexer's full-width logits): for each
// request, the min(k, L) positions of logits[0:L) with the largest scores,
// larger score first and the lower position first among equal scores, listed
// in ascending position order and padded with -1. Unlike the top-k the pages
// describe, it never touches positions at or past L, so its cost follows the
// actual length too.
//
// One 1024-lane workgroup per request runs an exact MSB-first radix select on
// order-preserving 32-bit keys: four passes of 8-bit digits, each building a
// 256-bin histogram (one private copy per wave in LDS, to keep atomics of
// different waves apart) of the keys that still match the digits fixed so far,
// then picking the bin that holds the k-th largest key. After the fourth pass
// the k-th largest key T and the number r of keys equal to T still needed are
// known exactly; a block-wide scan in position order then takes every key > T
// and the first r keys == T. Rows up to kLdsKeys positions keep their keys in
// LDS for all five sweeps; longer rows re-read the logits from memory.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 256;
constexpr int kLdsKeys = 32768;  // 128 KiB of keys

// Monotone map float -> uint32: a > b as floats (with -0 == +0) iff key(a) >
// key(b); NaN maps to 0, below the key of every number (-inf maps to 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (x == 0.0f) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (x != x) ? 0u : key;
}

__device__ __forceinline__ float load_f32(rsrc_t r, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
}
__device__ __forceinline__ void store_b32(rsrc_t r, int i, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, i * 4, 0, 0);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ seq_lens,
                                                         int32_t max_c4, int32_t k,
                                                         int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_vals) {
  __shared__ uint32_t keys[kLdsKeys];
  __shared__ uint32_t hist[kWaves][kBins];
  __shared__ uint32_t part[2 * kWaves];
  __shared__ uint32_t pick[2];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const uint64_t below = (1ull << lane) - 1ull;  // lanes with a smaller index
  const int len = min(max(seq_lens[b], 0), max_c4);
  // only positions [0, len) of the row are readable through this resource
  const rsrc_t row = make_rsrc(logits + (int64_t)b * max_c4, (uint32_t)len * 4u);
  const rsrc_t oi = make_rsrc(out_idx + (int64_t)b * k, (uint32_t)k * 4u);
  const bool with_vals = out_vals != nullptr;
  const rsrc_t ov = make_rsrc(with_vals ? static_cast<const void*>(out_vals + (int64_t)b * k) : out_idx,
                              with_vals ? (uint32_t)k * 4u : 0u);

  if (len <= k) {
    // every valid position is chosen
    for (int i = tid; i < k; i += kThreads) {
      store_b32(oi, i, i < len ? (uint32_t)i : 0xFFFFFFFFu);
      if (with_vals) store_b32(ov, i, i < len ? __builtin_bit_cast(uint32_t, load_f32(row, i)) : 0x7FC00000u);
    }
    return;
  }

  const bool cached = len <= kLdsKeys;
  if (cached) {
    for (int i = tid; i < len; i += kThreads) keys[i] = order_key(load_f32(row, i));
  }

  uint32_t prefix = 0, mask = 0;
  uint32_t remaining = (uint32_t)k;  // how many of the keys matching `prefix` are still to take
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kWaves * kBins; i += kThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < len; i += kThreads) {
      const uint32_t key = cached ? keys[i] : order_key(load_f32(row, i));
      if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // threads 0..255 (waves 0..3) own one bin each: total count, then the
    // suffix sum over bins >= own bin
    uint32_t cnt = 0, incl = 0;
    if (tid < kBins) {
      for (int wv = 0; wv < kWaves; ++wv) cnt += hist[wv][tid];
      incl = cnt;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_down(incl, off);
        if (lane + off < 64) incl += t;
      }
      if (lane == 0) part[wave] = incl;  // this wave's 64 bins
    }
    __syncthreads();
    if (tid < kBins) {
      for (int wv = wave + 1; wv < kBins / 64; ++wv) incl += part[wv];
      const uint32_t above = incl - cnt;  // keys in higher bins
      if (above < remaining && incl >= remaining) {
        pick[0] = (uint32_t)tid;
        pick[1] = above;
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= 255u << shift;
    remaining -= pick[1];
  }
  const uint32_t T = prefix;  // the k-th largest key; take `remaining` of its copies

  // selection in position order, 1024 positions per round
  uint32_t eq_seen = 0, written = 0;
  for (int start = 0; start < len && written < (uint32_t)k; start += kThreads) {
    const int i = start + tid;
    const uint32_t key = (i < len) ? (cached ? keys[i] : order_key(load_f32(row, i))) : 0u;
    const bool in = i < len;
    const bool gt = in && key > T;
    const bool eq = in && key == T;
    const uint64_t eq_mask = __ballot(eq);
    if (lane == 0) part[wave] = __popcll(eq_mask);
    __syncthreads();
    uint32_t eq_rank = eq_seen + __popcll(eq_mask & below), eq_total = 0;
    for (int wv = 0; wv < kWaves; ++wv) {
      const uint32_t c = part[wv];
      eq_rank += wv < wave ? c : 0u;
      eq_total += c;
    }
    const bool take = gt || (eq && eq_rank < remaining);
    const uint64_t take_mask = __ballot(take);
    if (lane == 0) part[kWaves + wave] = __popcll(take_mask);
    __syncthreads();
    uint32_t pos = written + __popcll(take_mask & below), take_total = 0;
    for (int wv = 0; wv < kWaves; ++wv) {
      const uint32_t c = part[kWaves + wv];
      pos += wv < wave ? c : 0u;
      take_total += c;
    }
    if (take) {  // exactly k are taken; pos < k
      store_b32(oi, (int)pos, (uint32_t)i);
      if (with_vals) store_b32(ov, (int)pos, __builtin_bit_cast(uint32_t, load_f32(row, i)));
    }
    eq_seen += eq_total;
    written += take_total;
    __syncthreads();  // `part` is rewritten next round
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                       int32_t k, int32_t* out_idx, float* out_vals, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kThreads), 0, stream, logits, seq_lens, max_c4, k,
                     out_idx, out_vals);
  return hipGetLastError();
}

}  // namespace dsa
