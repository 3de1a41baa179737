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
// One 1024-lane workgroup per request works on order-preserving 32-bit keys
// (larger float <=> larger key). Lane t holds the 32 consecutive positions
// [32 t, 32 t + 32) of a block of kBlock = 32768 positions in registers, read
// with eight 16-byte loads that are all in flight together.
//
// Candidate path (a row of one block): a row of at most kCap positions is its
// own candidate set; a longer row counts one sampled key per lane into a
// 2048-bin histogram of the top 11 key bits, and the lower edge of the bin
// holding a generous estimate of the k-th largest sample becomes a cut. The
// keys >= cut are counted exactly; if there are at least k (so every key of
// the top k is among them) and at most kCap, each lane writes its candidates
// (key, position) to LDS at an offset from one block-wide scan, which keeps
// them in position order. An exact MSB-first radix select with digits of 11,
// 11 and 10 bits over the candidates gives the k-th largest key T and r, the
// number of keys == T in the top k: each pass counts the candidates matching
// the digits fixed so far into a 2048-bin LDS histogram, and a block-wide scan
// over the bins, two per lane from the top bin down, finds the bin holding the
// k-th largest.
//
// Full path (a longer row, or a cut that missed): the same radix select over
// every key, re-reading the row block by block, out of line so that its
// registers are allocated apart from the candidate path's.
//
// Both paths place the chosen positions with one scan: before any point in
// position order, (keys > T before it) + min(r, keys == T before it) positions
// are taken, so a scan of the two counts packed in one word gives every lane
// its output offset. Values are rebuilt from the keys (-0 is reported as +0,
// any NaN as one NaN pattern). Wave-level scans use DPP row shifts and row
// broadcasts.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;                      // 11-bit digits
constexpr int kHistWords = kBins + kBins / 32;   // one pad word per 32 bins
constexpr int kPerLane = 32;                     // consecutive positions per lane
constexpr int kBlock = kPerLane * kThreads;      // 32768 positions per block
constexpr int kCap = 8192;                       // candidates held in LDS
constexpr uint32_t kNoPick = 0xFFFFFFFFu;

// Monotone map float -> uint32: a > b as floats (with -0 == +0) iff key(a) >
// key(b). Non-negative floats get the sign bit set, negative ones are
// complemented; NaN maps to 1, below the key of every number (-inf maps to
// 0x007FFFFF). Key 0 marks an unused slot past the row's length, so a key is
// valid iff it is >= 1.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);  // -0 + 0 = +0
  const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return (x != x) ? 1u : key;
}
// The float a key came from (+0 for either zero, a NaN for key 1).
__device__ __forceinline__ uint32_t key_to_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
}

__device__ __forceinline__ uint32_t load_b32(rsrc_t r, int i) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
}
__device__ __forceinline__ void store_b32(rsrc_t r, int i, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, i * 4, 0, 0);
}

// Digit of a key in pass p (0, 1, 2): bits 31..21, 20..10, 9..0.
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x3FFu : 0x7FFu; }
// LDS word of histogram bin b (a pad word after every 32 bins).
__device__ __forceinline__ int hist_word(uint32_t b) { return (int)(b + (b >> 5)); }

// Inclusive scan over the 64 lanes of a wave: row shifts by 1, 2, 4, 8 scan
// each row of 16 lanes, then row broadcasts of lanes 15 and 31 carry the row
// totals forward.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Inclusive scan of v over the block's lanes in lane order, and the block
// total; `part` is kWaves words of LDS scratch (16-byte aligned). Every lane
// of the block must call it.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* part, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  v = wave_inclusive_scan(v);
  if (lane == 63) part[wave] = v;
  __syncthreads();
  const u32x4* p4 = reinterpret_cast<const u32x4*>(part);
  uint32_t add = 0, all = 0;
#pragma unroll
  for (int q = 0; q < kWaves / 4; ++q) {
    const u32x4 w4 = p4[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      add += (4 * q + e < wave) ? w4[e] : 0u;
      all += w4[e];
    }
  }
  __syncthreads();
  *total = all;
  return v + add;
}

// The bin holding the rank-th largest of the counted keys, rank =
// rank_of(total counted): returns {bin, keys in higher bins, total}, or
// {kNoPick, total, total} if rank exceeds the total.
struct Pick {
  uint32_t bin, above, total;
};
template <typename RankOf>
__device__ __forceinline__ Pick pick_bin(const uint32_t* h, RankOf rank_of, uint32_t* part, uint32_t* pick) {
  const int tid = threadIdx.x;
  // lane t owns bins 2047-2t and 2046-2t, so a lane-order scan runs from the top bin down
  const uint32_t hi = (uint32_t)(kBins - 1 - 2 * tid), lo = hi - 1;
  const uint32_t h_hi = h[hist_word(hi)], h_lo = h[hist_word(lo)];
  uint32_t total;
  const uint32_t incl = block_inclusive_scan(h_hi + h_lo, part, &total);  // keys in bins >= lo
  const uint32_t rank = rank_of(total);
  const uint32_t above_hi = incl - h_lo - h_hi;                            // keys in bins > hi
  if (above_hi < rank && above_hi + h_hi >= rank) {
    pick[0] = hi;
    pick[1] = above_hi;
  } else if (above_hi + h_hi < rank && incl >= rank) {
    pick[0] = lo;
    pick[1] = above_hi + h_hi;
  } else if (tid == 0 && rank > total) {
    pick[0] = kNoPick;
    pick[1] = total;
  }
  __syncthreads();
  Pick p{pick[0], pick[1], total};
  __syncthreads();  // pick[] is rewritten by the next call
  return p;
}

// LDS of the kernel, at namespace scope so the out-of-line full path reaches
// it with LDS instructions too.
__shared__ uint32_t hist[2][kHistWords];  // counted into alternately
__shared__ uint32_t cand_key[kCap];
__shared__ uint32_t cand_pos[kCap];
__shared__ __attribute__((aligned(16))) uint32_t part[kWaves];
__shared__ uint32_t pick[2];

// Keys of the block at `blk` into this lane's registers: key[j] is position
// blk + 32 * lane + j; slots at or past len get key 0. With at least k valid
// keys (the row is longer than k), the k-th largest key is a valid one, so a
// key-0 slot never reaches a bin at or above it and is never taken.
__device__ __forceinline__ void load_block(rsrc_t row, bool vec, int blk, int len, uint32_t (&key)[kPerLane]) {
  const int base = blk + kPerLane * (int)threadIdx.x;
  const int n = min(max(len - base, 0), kPerLane);
  if (vec && n == kPerLane) {
    u32x4 v[kPerLane / 4];
#pragma unroll
    for (int m = 0; m < kPerLane / 4; ++m) v[m] = __builtin_amdgcn_raw_buffer_load_b128(row, (base + 4 * m) * 4, 0, 0);
#pragma unroll
    for (int m = 0; m < kPerLane / 4; ++m) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // element first, then reinterpret (a bit_cast of a vector-element
        // lvalue reads element 0 whatever the index)
        const uint32_t bits = v[m][e];
        key[4 * m + e] = order_key(__uint_as_float(bits));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
      key[j] = j < n ? order_key(__uint_as_float(load_b32(row, base + j))) : 0u;
  }
}

// Full path: exact radix select over every key of the row, re-reading the row
// block by block in every sweep.
__device__ __noinline__ void full_path(rsrc_t row, rsrc_t oi, rsrc_t ov, bool with_vals, bool vec, int len,
                                       int k) {
  const int tid = threadIdx.x;
  uint32_t key[kPerLane];
  for (int i = tid; i < 2 * kHistWords; i += kThreads) (&hist[0][0])[i] = 0u;
  __syncthreads();
  int cur = 0;
  uint32_t T = 0u, mask = 0u, remaining = (uint32_t)k;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = digit_shift(pass);
    const uint32_t dmask = digit_mask(pass);
    for (int blk = 0; blk < len; blk += kBlock) {
      load_block(row, vec, blk, len, key);
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const uint32_t kk = key[j];
        if ((kk & mask) == T) atomicAdd(&hist[cur][hist_word((kk >> shift) & dmask)], 1u);
      }
    }
    __syncthreads();
    for (int i = tid; i < kHistWords; i += kThreads) hist[cur ^ 1][i] = 0u;
    const Pick p = pick_bin(hist[cur], [&](uint32_t) { return remaining; }, part, pick);
    cur ^= 1;
    T |= p.bin << shift;
    remaining -= p.above;
    mask |= dmask << shift;
  }
  uint32_t gt_seen = 0, eq_seen = 0;  // block-uniform totals over earlier blocks
  for (int blk = 0; blk < len; blk += kBlock) {
    load_block(row, vec, blk, len, key);
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      n_gt += key[j] > T ? 1u : 0u;
      n_eq += key[j] == T ? 1u : 0u;
    }
    const uint32_t packed = (n_gt << 16) | n_eq;  // block totals < 2^16: no carry
    uint32_t blk_tot;
    const uint32_t before = block_inclusive_scan(packed, part, &blk_tot) - packed;
    uint32_t eq_rank = eq_seen + (before & 0xFFFFu);
    uint32_t pos = gt_seen + (before >> 16) + min(remaining, eq_rank);
    if (n_gt + n_eq != 0) {
      const int base = blk + kPerLane * tid;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const bool gt = key[j] > T, eq = key[j] == T;
        if (gt || (eq && eq_rank < remaining)) {
          store_b32(oi, (int)pos, (uint32_t)(base + j));
          if (with_vals) store_b32(ov, (int)pos, key_to_bits(key[j]));
          ++pos;
        }
        eq_rank += eq ? 1u : 0u;
      }
    }
    gt_seen += blk_tot >> 16;
    eq_seen += blk_tot & 0xFFFFu;
  }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ seq_lens,
                                                         int32_t max_c4, int32_t k,
                                                         int32_t* __restrict__ out_idx,
                                                         float* __restrict__ out_vals) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = min(max(seq_lens[b], 0), max_c4);
  const float* row_ptr = logits + (int64_t)b * max_c4;
  // only positions [0, len) of the row are readable through this resource
  const rsrc_t row = make_rsrc(row_ptr, (uint32_t)len * 4u);
  const rsrc_t oi = make_rsrc(out_idx + (int64_t)b * k, (uint32_t)k * 4u);
  const bool with_vals = out_vals != nullptr;
  const rsrc_t ov = make_rsrc(with_vals ? static_cast<const void*>(out_vals + (int64_t)b * k) : out_idx,
                              with_vals ? (uint32_t)k * 4u : 0u);

  if (len <= k) {
    // every valid position is chosen
    for (int i = tid; i < k; i += kThreads) {
      store_b32(oi, i, i < len ? (uint32_t)i : 0xFFFFFFFFu);
      if (with_vals) store_b32(ov, i, i < len ? load_b32(row, i) : 0x7FC00000u);
    }
    return;
  }
  const bool vec = (reinterpret_cast<uintptr_t>(row_ptr) & 15u) == 0;

  if (len <= kBlock) {
    uint32_t key[kPerLane];
    load_block(row, vec, 0, len, key);
    uint32_t cut = 1u;  // candidates: keys >= cut (1: every valid key)
    bool ok = len <= kCap;
    if (!ok && k <= kCap) {
      for (int i = tid; i < kHistWords; i += kThreads) hist[0][i] = 0u;
      __syncthreads();
      // one sampled key per lane, spread over the lane's run
      const int js = tid & (kPerLane - 1);
      uint32_t ks = 0u;  // key[js] without a lane-varying register index
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) ks = j == js ? key[j] : ks;
      if (ks != 0u) atomicAdd(&hist[0][hist_word(ks >> 21)], 1u);
      __syncthreads();
      // aim 25% (+16 samples) above the expected number of sampled keys in the top k
      const Pick p = pick_bin(hist[0], [&](uint32_t n) {
        return (uint32_t)(((uint64_t)k * n * 5u) / (4u * (uint64_t)len)) + 16u; }, part, pick);
      ok = p.bin != kNoPick && p.bin != 0u;
      cut = ok ? p.bin << 21 : 1u;
    }
    // candidates of this lane, as a bit mask over its run
    uint32_t cm = 0u;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) cm |= (key[j] >= cut ? 1u : 0u) << j;
    uint32_t n_cand;
    const uint32_t mine = (uint32_t)__popc(cm);
    uint32_t at = block_inclusive_scan(mine, part, &n_cand) - mine;
    if (ok || n_cand <= (uint32_t)kCap) ok = n_cand >= (uint32_t)k && n_cand <= (uint32_t)kCap;
    if (ok) {
      const int base = kPerLane * tid;
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        if (cm & (1u << j)) {
          cand_key[at] = key[j];
          cand_pos[at] = (uint32_t)(base + j);
          ++at;
        }
      }
      for (int i = tid; i < 2 * kHistWords; i += kThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();

      // exact radix select over the candidates
      int cur = 0;
      uint32_t T = 0u, mask = 0u, remaining = (uint32_t)k;
      for (int pass = 0; pass < 3; ++pass) {
        const int shift = digit_shift(pass);
        const uint32_t dmask = digit_mask(pass);
        for (int i = tid; i < (int)n_cand; i += kThreads) {
          const uint32_t kk = cand_key[i];
          if ((kk & mask) == T) atomicAdd(&hist[cur][hist_word((kk >> shift) & dmask)], 1u);
        }
        __syncthreads();
        for (int i = tid; i < kHistWords; i += kThreads) hist[cur ^ 1][i] = 0u;
        const Pick p = pick_bin(hist[cur], [&](uint32_t) { return remaining; }, part, pick);
        cur ^= 1;
        T |= p.bin << shift;
        remaining -= p.above;
        mask |= dmask << shift;
      }

      // each lane takes a run of consecutive candidates
      const int per = ((int)n_cand + kThreads - 1) / kThreads;  // <= kCap / kThreads
      const int c0 = min(tid * per, (int)n_cand), c1 = min(c0 + per, (int)n_cand);
      uint32_t n_gt = 0, n_eq = 0;
      for (int i = c0; i < c1; ++i) {
        const uint32_t kk = cand_key[i];
        n_gt += kk > T ? 1u : 0u;
        n_eq += kk == T ? 1u : 0u;
      }
      const uint32_t packed = (n_gt << 16) | n_eq;
      uint32_t unused;
      const uint32_t before = block_inclusive_scan(packed, part, &unused) - packed;
      uint32_t eq_rank = before & 0xFFFFu;
      uint32_t pos = (before >> 16) + min(remaining, eq_rank);
      for (int i = c0; i < c1; ++i) {
        const uint32_t kk = cand_key[i];
        if (kk > T || (kk == T && eq_rank < remaining)) {
          store_b32(oi, (int)pos, cand_pos[i]);
          if (with_vals) store_b32(ov, (int)pos, key_to_bits(kk));
          ++pos;
        }
        eq_rank += kk == T ? 1u : 0u;
      }
      return;
    }
  }
  full_path(row, oi, ov, with_vals, vec, len, k);
}

}  // namespace

hipError_t launch_topk(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                       int32_t k, int32_t* out_idx, float* out_vals, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kThreads), 0, stream, logits, seq_lens, max_c4, k,
                     out_idx, out_vals);
  return hipGetLastError();
}

}  // namespace dsa
