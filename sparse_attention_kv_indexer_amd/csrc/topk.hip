// Top-k of the DSA indexer decode step on gfx950.
//
// What it computes (page "The O(Actual) Indexer", section "The Benchmark
// Results": the top-k that consumes the indexer's full-width logits): for each
// request, the min(k, L) positions of logits[0:L) with the largest scores,
// larger score first and the lower position first among equal scores, listed
// in ascending position order and padded with -1. Unlike the top-k the pages
// describe, it never touches positions at or past L, so its cost follows the
// actual length too.
//
// Keys. Scores become order-preserving 32-bit keys (larger float <=> larger
// key; -0 and +0 equal; NaN below -inf). The k-th largest key T is found by an
// exact MSB-first radix select with digits of 11, 11 and 10 bits; r is the
// number of keys == T that belong to the top k (the lowest positions first).
// Before any point in position order, (keys > T before it) + min(r, keys == T
// before it) positions are taken, so counting those two kinds of keys in
// position order places every chosen position. (A row held in registers whose
// cut lies above +0 keeps its candidates as the raw score bits instead: every
// one is a positive float or +inf, whose bits order as the keys do.)
//
// One 1024-lane workgroup per request (the row kernel) selects its row's top
// k. Every row of at most kSeg positions is its own candidate set, read
// straight from the logits. A longer row is cut to candidates first: the keys
// at or above a cut, with their positions, in position order in LDS. The
// exact radix select then runs over the candidates at or above the cut only,
// on digits of their offset from it (a narrow key range, so the first pass
// spreads over many bins). If T lies below the cut (fewer than k keys reach
// it) or more candidates remain than LDS holds, the workgroup selects over
// the whole row instead, re-reading it from memory, so a cut never changes
// the result. Where the cut and the candidates come from depends on the row
// width:
//  * Row width at most kRes (one kernel, no workspace): the workgroup loads
//    the whole row into registers, cuts it at a key sampled from 64 runs of
//    32 positions (loaded first, so the cut is picked while the row arrives),
//    and each wave stores its chunk's kept keys to its own region of LDS as
//    they arrive (gather_resident).
//  * Wider rows (two kernels, so that no workgroup waits on another one): a
//    segment kernel (rows longer than kSeg positions only; grid: requests x
//    at most kSegGridY (8), 256 lanes, each workgroup taking every
//    kSegGridY-th segment) cuts each segment of kSeg positions at the lower
//    edge of the bin holding a generous estimate of the segment's share of
//    the top k (from two sampled keys per lane), and each wave writes its
//    kept keys with their positions, in position order, to its own sub-slot
//    of the workspace, with its count. The row kernel gathers the sub-slots
//    into LDS in order, hence position order (the first kSpec pairs of the
//    first kSpecSlots sub-slots are loaded together with the counts, before
//    the counts are known); the largest segment cut serves as the cut: if T
//    is at or above every segment's cut, each key a segment left out is below
//    T.
//
// With the score kernel's first-digit histogram of the row (the fused pair),
// the cut is the exact lower edge of the bin holding the k-th largest key
// (for every segment, or for the row held in registers), the row kernel
// starts its select at the second digit, and it sets the histogram back to
// zero.
//
// A radix pass counts into a histogram in LDS; four waves of the row kernel,
// one per SIMD, then pick the digit (block_pick; in the segment kernel every
// wave reads the whole histogram itself, which spares a broadcast).
#include "common.h"

namespace dsa {
namespace {

constexpr int kBins = 2048;  // 11-bit digits (the last digit has 10 bits)

constexpr int kSegThreads = 256;              // segment kernel
constexpr int kSegWaves = kSegThreads / 64;
constexpr int kSeg = 4096;                    // positions per segment workgroup
constexpr int kPerLane = kSeg / kSegThreads;  // 16 consecutive positions per lane
constexpr int kSub = kSeg / kSegWaves;        // 1024 positions per wave: one sub-slot
// Segment workgroups per request: each takes segments y, y + kSegGridY, ...
// Rows of up to 8 segments (a 128K-token row width) get one workgroup per
// segment; a wider row width launches no more workgroups that only read a
// short length and exit (measured at a 1M-token width with 512-token lengths:
// cap 32 -> 8, top-k 7.24 -> 7.02 us; cap 4 makes 128K rows 2.4 us slower).
constexpr int kSegGridY = 8;
constexpr int kRecWords = 8;                  // per segment: kept count of each wave, cut key, unused

constexpr int kRowThreads = 1024;             // row kernel
constexpr int kRowWaves = kRowThreads / 64;
static_assert(kRowWaves == 16, "wave_partials: one wave's totals per lane of a 16-lane DPP row");
// LDS words of cand_key and of cand_pos each: 16320 puts cand_pos[i]
// exactly 255 x 256 bytes past cand_key[i], so that one ds_write2st64_b32
// stores a key and its position from one address (two separate stores cost
// c3 top-k 13.91 vs 13.69 us, A/B on one box).
constexpr int kSlots = 16320;
constexpr int kCap = kSlots - kRowThreads;    // candidates the row workgroup of the widest rows holds in LDS
constexpr int kRound = 256;                   // sub-slot records per gather round
constexpr int kSpecSlots = 32;                // sub-slots read before their counts are known
constexpr int kSpec = 256;                    // pairs read ahead per such sub-slot
constexpr int kSweep = 16 * kRowThreads;      // positions per block of the whole-row output sweep
constexpr int kSmall = 64;                    // keys of a bin that one wave ranks directly
constexpr int kSmallRanged = 16;              // the same, in the ranged select over long rows' candidates
// A row width of at most kRes positions needs no segment kernel: the row
// kernel holds a whole row in registers (kResBlk blocks of kSeg positions,
// four consecutive positions of each per lane) and cuts it itself, from
// kSamples keys in 64 runs of 32 consecutive positions spread over the row.
constexpr int kRes = 32768;
constexpr int kResBlk = kRes / kSeg;
// In that kernel each wave keeps its candidates in a region of its own:
// wave w's at slots [w kRegion, w kRegion + its count), so that it stores
// them as its keys arrive, with no workgroup-wide scan.
constexpr int kRegion = kSlots / kRowWaves;
constexpr uint32_t kOverflow = 1u << 16;  // added to the candidate count for a region that overflowed
static_assert(kRowWaves * kRegion + 3 * 64 <= 2 * kSlots, "the count's reads past a region stay in cand_pos");
constexpr int kSamples = 2 * kRowThreads;     // the sample: 64 runs of 32 positions
static_assert(kSeg == 4 * kRowThreads, "a block of kSeg positions is one 16-byte group per lane");
static_assert(2 * kBins <= kCap, "the sample histograms fit in cand_pos");
static_assert(kCap + 3 * kRowThreads <= 2 * kSlots, "the ranged count's reads past n stay in cand_pos");

static_assert(kSegWaves * 64 == kSegThreads && kPerLane * kSegThreads == kSeg, "segment work split");
static_assert(2 * kRowThreads * 4 == kSpecSlots * kSpec, "read-ahead: four 16-byte loads per lane");
static_assert(kBins == kHistBins && kHistShift == 21, "the score kernel's histogram is the first radix digit");

// The float a key came from (+0 for either zero, a NaN for key 1).
__device__ __forceinline__ uint32_t key_to_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t load_b32(rsrc_t r, int i) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
}
__device__ __forceinline__ void store_b32(rsrc_t r, int i, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, i * 4, 0, 0);
}
// Pair i (words 2i, 2i + 1) of a buffer of pairs.
__device__ __forceinline__ u32x2 load_pair(rsrc_t r, int i) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, i * 8, 0, 0);
}
__device__ __forceinline__ void store_pair(rsrc_t r, int i, uint32_t a, uint32_t b) {
  u32x2 v;
  v.x = a;
  v.y = b;
  __builtin_amdgcn_raw_buffer_store_b64(v, r, i * 8, 0, 0);
}

// LDS word of histogram bin b. Within each group of 32 bins the eight 4-bin
// chunks are permuted by the group index, so that the lanes of a wave, each
// reading its own group chunk by chunk, spread over the LDS banks.
__device__ __forceinline__ uint32_t hslot(uint32_t b) { return b ^ (((b >> 5) & 7u) << 2); }

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

// The largest value over the 64 lanes of a wave, in every lane: the same DPP
// steps as the scan with max (0 is neutral), then lane 63's value.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The second half of a block scan over the 16 waves of a row workgroup: wave
// w's kN (<= 4) wave totals sit at part[4w .. 4w + kN - 1], 16-byte aligned
// (written by its lane 63, then a barrier). Every lane gets, for each q, the
// sum over the waves before its own and the sum over all: each 16-lane row
// of the wave takes one wave's totals per lane, scans them along the row
// (DPP row shifts), and the two sums are read from lanes wave - 1 and 15.
// (Each wave adding all 16 waves' totals itself took about 100 instructions
// per wave for four values, where this takes about 30.)
template <int kN>
__device__ __forceinline__ void wave_partials(const uint32_t* part, uint32_t (&before)[kN], uint32_t (&all)[kN]) {
  static_assert(kN <= 4, "four values per wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // 0 .. 15
  const u32x4 p = *reinterpret_cast<const u32x4*>(part + 4 * (lane & 15));
#pragma unroll
  for (int q = 0; q < kN; ++q) {
    uint32_t v = p[q];
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    const uint32_t prev = (uint32_t)__builtin_amdgcn_readlane((int)v, max(wave - 1, 0));
    before[q] = wave > 0 ? prev : 0u;
    all[q] = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  }
}

// Inclusive scans of a and b over the row workgroup's lanes in lane order,
// and their totals; `part` is 4 * 16 words of LDS, 16-byte aligned. Every
// lane must call it; it ends with a barrier, after which part may be
// rewritten.
__device__ __forceinline__ void block_scan2(uint32_t& a, uint32_t& b, uint32_t* part, uint32_t* tot_a, uint32_t* tot_b) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  a = wave_inclusive_scan(a);
  b = wave_inclusive_scan(b);
  if (lane == 63) {
    part[4 * wave] = a;
    part[4 * wave + 1] = b;
  }
  __syncthreads();
  uint32_t before[2], all[2];
  wave_partials<2>(part, before, all);
  __syncthreads();
  a += before[0];
  b += before[1];
  *tot_a = all[0];
  *tot_b = all[1];
}

// From a histogram of kNB bins in LDS (complete, after a barrier), the bin
// holding the rank-th largest counted key (rank = rank_of(total counted) >=
// 1) and the number of counted keys in higher bins; {0, total} if rank
// exceeds the total. Called by whole waves; each wave reads every bin and
// finds the answer itself (lane l owns the kNB / 64 bins just below the top
// kNB / 64 * l), so no barrier or broadcast follows.
struct Pick {
  uint32_t bin, above;
  bool ok;  // false: the histogram holds fewer keys than the rank asked for
};
// load4(q, b) returns bins b .. b + 3 (b = the lane's lowest bin + 4 q).
template <int kNB>
__device__ __forceinline__ uint32_t pick_lo() {
  return (uint32_t)(kNB - (kNB / 64) * ((threadIdx.x & 63) + 1));  // the lane's lowest bin
}
template <int kNB, typename Load4, typename RankOf>
__device__ __forceinline__ Pick wave_pick(Load4 load4, RankOf rank_of) {
  constexpr int kPer = kNB / 64;    // bins per lane
  constexpr int kChunks = kPer / 4;
  const uint32_t lo = pick_lo<kNB>();
  uint32_t c[kPer];
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    const u32x4 v = load4(q, lo + 4 * q);  // bins lo + 4q .. + 3
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = v[e];
      c[4 * q + e] = x;
    }
  }
  uint32_t cs[kChunks], s = 0;
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
    cs[q] = c[4 * q] + c[4 * q + 1] + c[4 * q + 2] + c[4 * q + 3];
    s += cs[q];
  }
  const uint32_t incl = wave_inclusive_scan(s);
  const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
  const uint32_t rank = rank_of(total);
  const uint32_t excl = incl - s;
  const uint64_t hit = __ballot(excl < rank && rank <= incl);
  if (hit == 0) return Pick{0u, total, false};
  const int src = __builtin_ctzll(hit);
  // in the lane holding it: the chunk, top chunk first, then the bin
  uint32_t acc = excl, above_q = 0;
  int qs = 0;
  bool done = false;
#pragma unroll
  for (int q = kChunks - 1; q >= 0; --q) {
    if (!done && acc + cs[q] >= rank) {
      qs = q;
      above_q = acc;
      done = true;
    }
    acc += cs[q];
  }
  uint32_t e4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < kChunks; ++q) {
#pragma unroll
    for (int e = 0; e < 4; ++e) e4[e] = q == qs ? c[4 * q + e] : e4[e];
  }
  acc = above_q;
  uint32_t bin = 0, above = 0;
  done = false;
#pragma unroll
  for (int e = 3; e >= 0; --e) {
    if (!done && acc + e4[e] >= rank) {
      bin = lo + 4u * (uint32_t)qs + (uint32_t)e;
      above = acc;
      done = true;
    }
    acc += e4[e];
  }
  return Pick{(uint32_t)__builtin_amdgcn_readlane((int)bin, src), (uint32_t)__builtin_amdgcn_readlane((int)above, src),
              true};
}

// wave_pick over a histogram in LDS (bins at hslot positions).
template <int kNB, typename RankOf>
__device__ __forceinline__ Pick wave_pick_lds(const uint32_t* hist, RankOf rank_of) {
  return wave_pick<kNB>([&](int, uint32_t b) { return *reinterpret_cast<const u32x4*>(hist + hslot(b)); },
                        rank_of);
}

// The score kernel's first-digit histogram of row b, loaded in wave_pick's
// order (chunk q of the lane's bins); the loads are only issued here.
struct HistRegs {
  u32x4 c[kBins / 64 / 4];
};
__device__ __forceinline__ HistRegs load_row_hist(const uint32_t* hist, int b) {
  const rsrc_t hr = make_rsrc(hist + (size_t)b * kHistBins, kHistBins * 4u);
  const uint32_t lo = pick_lo<kBins>();
  HistRegs h;
#pragma unroll
  for (int q = 0; q < kBins / 64 / 4; ++q)
    h.c[q] = __builtin_amdgcn_raw_buffer_load_b128(hr, (lo + 4 * q) * 4, 0, 0);
  return h;
}
// The bin of the k-th largest key of the row and the count above it.
__device__ __forceinline__ Pick pick_row_hist(const HistRegs& h, int k) {
  return wave_pick<kBins>([&](int q, uint32_t) { return h.c[q]; }, [&](uint32_t) { return (uint32_t)k; });
}

// Workspace layout (32-bit words), for B requests and n_seg segments per row:
//   rec   [B][n_seg][kRecWords]           kept count of waves 0..3, cut key, unused
//   pairs [B][n_seg][kSegWaves][kSub][2]  kept (key, position) of each wave, in position order
__device__ __forceinline__ size_t ws_pairs(int b, int batch, int n_seg) {
  return (size_t)batch * n_seg * kRecWords + (size_t)b * n_seg * 2 * kSeg;
}

// ---------------------------------------------------------------------------
// Segment kernel
// ---------------------------------------------------------------------------

struct SegShared {
  __attribute__((aligned(16))) uint32_t hist[kBins];
};

// One segment (seg) of request b's row of len positions (kSeg < len, k < len).
// With the score kernel's histogram (hist != nullptr) the cut is exact: the
// lower edge of the bin holding the row's k-th largest key, the same for every
// segment of the row.
__device__ __forceinline__ void process_segment(SegShared& sm, const float* __restrict__ logits, int b, int seg,
                                                int len, int max_c4, int k, int n_seg, int batch,
                                                uint32_t* __restrict__ ws, const uint32_t* __restrict__ hist) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  HistRegs hr;
  if (hist != nullptr) hr = load_row_hist(hist, b);  // in flight with the row's loads
  const int s0 = seg * kSeg;
  const float* row_ptr = logits + (int64_t)b * max_c4;
  // only positions [0, len) of the row are readable through this resource
  const rsrc_t row = make_rsrc(row_ptr, (uint32_t)len * 4u);
  const int base = s0 + kPerLane * tid;
  const int n = min(max(len - base, 0), kPerLane);
  uint32_t key[kPerLane];
  if (n == kPerLane && (reinterpret_cast<uintptr_t>(row_ptr) & 15u) == 0) {
    u32x4 v[kPerLane / 4];
#pragma unroll
    for (int m = 0; m < kPerLane / 4; ++m)
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(row, (base + 4 * m) * 4, 0, 0);
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
    // every load is issued (past len the resource reads 0), then masked
    uint32_t bits[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) bits[j] = load_b32(row, base + j);
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) key[j] = j < n ? order_key(__uint_as_float(bits[j])) : 0u;
  }

  // The segment's expected share of the top k is k * valid / len; keep at
  // least 1.5 times that plus 32, judged from a 1-in-8 sample.
  const int valid = min(len - s0, kSeg);
  const float want = 1.5f * (float)k * ((float)valid / (float)len) + 32.0f;
  const uint32_t share = want < (float)valid ? (uint32_t)want : (uint32_t)valid;
  uint32_t cut = 1u;  // keep every valid key
  if (hist != nullptr) {
    // (a total below k cannot come from the same logits; it keeps every key)
    cut = max(pick_row_hist(hr, k).bin << 21, 1u);
  } else if (share < (uint32_t)valid) {
    for (int i = tid; i < kBins; i += kSegThreads) sm.hist[i] = 0u;
    __syncthreads();
    const int ja = tid & (kPerLane - 1), jb = (tid + kPerLane / 2) & (kPerLane - 1);
    uint32_t ka = 0u, kb = 0u;  // key[ja], key[jb] without a lane-varying register index
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
      ka = j == ja ? key[j] : ka;
      kb = j == jb ? key[j] : kb;
    }
    if (ka != 0u) atomicAdd(&sm.hist[hslot(ka >> 21)], 1u);
    if (kb != 0u) atomicAdd(&sm.hist[hslot(kb >> 21)], 1u);
    __syncthreads();
    // aim 25% (+4 samples) above the share among the samples
    const Pick p = wave_pick_lds<kBins>(sm.hist, [&](uint32_t n_s) {
      return (uint32_t)(1.25f * (float)share * ((float)n_s / (float)valid)) + 4u; });
    cut = max(p.bin << 21, 1u);
  }

  // this wave's kept keys, in position order, into its sub-slot
  uint32_t cm = 0u;  // this lane's kept keys, as a bit mask over its run
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) cm |= (key[j] >= cut ? 1u : 0u) << j;
  const uint32_t mine = (uint32_t)__popc(cm);
  const uint32_t incl = wave_inclusive_scan(mine);
  uint32_t at = incl - mine;
  uint32_t* pairs = ws + ws_pairs(b, batch, n_seg);
  const rsrc_t slot = make_rsrc(pairs + ((size_t)seg * kSegWaves + wave) * 2 * kSub, kSub * 8u);
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    if (cm & (1u << j)) {
      store_pair(slot, (int)at, key[j], (uint32_t)(base + j));
      ++at;
    }
  }
  const rsrc_t rec = make_rsrc(ws + ((size_t)b * n_seg + seg) * kRecWords, kRecWords * 4u);
  if (lane == 63) store_b32(rec, wave, incl);
  if (tid == 0) store_b32(rec, kSegWaves, cut);
}

// Grid: requests x segment groups; workgroup (b, y) takes segments y, y +
// gridDim.y, ... of request b's row. With the request index first, the
// workgroups of one row share b's place in the round-robin order of
// workgroups over the chip's XCDs when the batch is a multiple of 8, so they
// run on the XCD (and L2) where the row kernel's workgroup b, which reads
// their output, runs.
__global__ __launch_bounds__(kSegThreads) void topk_segment_kernel(const float* __restrict__ logits,
                                                                    const int32_t* __restrict__ seq_lens,
                                                                    int32_t max_c4, int32_t k, int32_t n_seg,
                                                                    uint32_t* __restrict__ ws,
                                                                    const uint32_t* __restrict__ hist) {
  __shared__ SegShared sm;
  const int b = blockIdx.x;
  const int len = min(max(seq_lens[b], 0), max_c4);
  if (len <= kSeg || len <= k) return;  // the row kernel handles such a row alone
  for (int seg = blockIdx.y; seg * kSeg < len; seg += gridDim.y) {
    process_segment(sm, logits, b, seg, len, max_c4, k, n_seg, (int)gridDim.x, ws, hist);
    __syncthreads();  // sm is reused by the next segment
  }
}

// ---------------------------------------------------------------------------
// Row kernel
// ---------------------------------------------------------------------------

// LDS of the row kernel, at namespace scope so the out-of-line whole-row path
// reaches it with LDS instructions too.
struct RowShared {
  // first, so that cand_pos[i] is cand_key[i]'s address plus 255 x 256
  // bytes, the largest second offset of ds_write2st64_b32
  __attribute__((aligned(16))) uint32_t cand_key[kSlots];
  __attribute__((aligned(16))) uint32_t cand_pos[kSlots];
  __attribute__((aligned(16))) uint32_t hist0[kBins];  // one histogram per radix pass
  __attribute__((aligned(16))) uint32_t hist1[kBins];
  __attribute__((aligned(16))) uint32_t hist2[kBins / 2];
  uint32_t cnt[kRound];   // per sub-slot of a gather round: kept count
  uint32_t off[kRound];   //   its first candidate
  uint32_t roff[kRound];  //   its first pair not read ahead, in the round's list of those
  __attribute__((aligned(16))) uint32_t part[4 * kRowWaves];  // four values per wave (wave_partials)
  uint32_t bcast[3];
  uint32_t hpick[3];  // from the score kernel's histogram: bin of the k-th largest, count above it, found
  __attribute__((aligned(16))) uint32_t small[kSmall];  // the keys of the last bin, once at most kSmall remain
  uint32_t small_n;
  uint32_t range[2];  // candidates at or above the largest cut, largest candidate key
  uint32_t max_cut;
  uint32_t dummy[64];  // per lane: where the ranged select's count adds a key it does not count
};
__shared__ RowShared rs;

__device__ __forceinline__ uint32_t* pass_hist(int pass) {
  return pass == 0 ? rs.hist0 : (pass == 1 ? rs.hist1 : rs.hist2);
}

// The candidate slots one lane visits, i = first, first + step, ... below
// end, at rs.cand_key[base + i]: in the resident kernel (each wave's
// candidates in its own region) the wave's lanes take its region, otherwise
// the workgroup's lanes take [0, n).
struct Slots {
  int base, first, end, step;
};
__device__ __forceinline__ Slots all_slots(int n) { return Slots{0, (int)threadIdx.x, n, kRowThreads}; }
__device__ __forceinline__ Slots region_slots(int count) {
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  return Slots{wave * kRegion, (int)(threadIdx.x & 63), count, 64};
}

// Clears the three histograms, max_cut and the last bin's key count (a
// barrier must follow before they are counted into).
__device__ __forceinline__ void clear_hists() {
  if (threadIdx.x == 0) {
    rs.small_n = 0u;
    rs.max_cut = 0u;
    rs.range[0] = 0u;
    rs.range[1] = 0u;
  }
  for (int i = threadIdx.x; i < kBins; i += kRowThreads) {
    rs.hist0[i] = 0u;
    rs.hist1[i] = 0u;
    if (i < kBins / 2) rs.hist2[i] = 0u;
  }
}

// The row kernel's pick over a histogram of kNB bins in LDS (complete, after
// a barrier): waves 0-3, one per SIMD, read the bins, kNB / 256 per lane (lane
// t the ones just below the top kNB / 256 * t), each scans its lanes' counts,
// the four wave totals go through LDS, and the one lane whose bins hold the
// rank-th largest counted key (rank = rank_of(total counted)) writes
// rs.bcast = {bin, keys in higher bins, keys in the bin} ({0, total, 0} if
// rank exceeds the total). The other waves only pass the barriers: a SIMD
// runs its waves one after another, so a pick spread over all 16 waves took
// four waves' worth of instructions per SIMD (about 0.6 us, and wave 0 alone
// over 32 bins per lane 0.75 us). Every lane must call it; it ends with a
// barrier, after which rs.bcast is read.
template <int kNB, typename RankOf>
__device__ __forceinline__ void block_pick(const uint32_t* h, RankOf rank_of) {
  constexpr int kPickWaves = 4;
  constexpr int kPer = kNB / (64 * kPickWaves);
  static_assert(kPer == 4 || kPer == 8, "four or eight bins per lane");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool picker = wave < kPickWaves;
  const uint32_t lo = (uint32_t)(kNB - kPer * (min(tid, 64 * kPickWaves - 1) + 1));  // this lane's lowest bin
  uint32_t c[kPer];
  uint32_t sum = 0u, incl = 0u;
  if (picker) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      // bins lo + 4q .. + 3: one 4-bin chunk, which hslot keeps in order
      const u32x4 v = *reinterpret_cast<const u32x4*>(h + hslot(lo + 4 * q));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = v[e];
        c[4 * q + e] = x;
        sum += x;
      }
    }
    incl = wave_inclusive_scan(sum);
    if (lane == 63) rs.part[wave] = incl;
  }
  __syncthreads();
  if (picker) {
    uint32_t pre = 0u, total = 0u;
#pragma unroll
    for (int w = 0; w < kPickWaves; ++w) {
      const uint32_t t = rs.part[w];
      pre += w < wave ? t : 0u;
      total += t;
    }
    const uint32_t rank = rank_of(total);
    const uint32_t excl = pre + incl - sum;
    if (excl < rank && rank <= excl + sum) {  // exactly one lane: its bins, highest first
      uint32_t acc = excl, bin = lo, above = excl, cnt = 0u;
      bool done = false;
#pragma unroll
      for (int e = kPer - 1; e >= 0; --e) {
        if (!done && acc + c[e] >= rank) {
          bin = lo + (uint32_t)e;
          above = acc;
          cnt = c[e];
          done = true;
        }
        acc += c[e];
      }
      rs.bcast[0] = bin;
      rs.bcast[1] = above;
      rs.bcast[2] = cnt;
    }
    if (tid == 0 && rank > total) {
      rs.bcast[0] = 0u;
      rs.bcast[1] = total;
      rs.bcast[2] = 0u;
    }
  }
  __syncthreads();
}

// Resolves one digit: counts the keys matching (T, mask) into pass's
// histogram with `count`; the workgroup picks the digit of the k-th largest
// (block_pick), which every lane then reads from LDS.
// Returns how many keys match the resolved digits (the count in the chosen bin).
template <int kPass, typename Count>
__device__ __forceinline__ uint32_t radix_pass(uint32_t& T, uint32_t& mask, uint32_t& remaining, Count count) {
  constexpr int shift = kPass == 0 ? 21 : (kPass == 1 ? 10 : 0);
  constexpr uint32_t dmask = kPass == 2 ? 0x3FFu : 0x7FFu;
  uint32_t* h = pass_hist(kPass);
  count(h, shift, dmask);
  __syncthreads();
  block_pick<(kPass == 2 ? kBins / 2 : kBins)>(h, [&](uint32_t) { return remaining; });
  // (bcast is written again only after the next pass's first barrier)
  T |= rs.bcast[0] << shift;
  remaining -= rs.bcast[1];
  mask |= dmask << shift;
  return rs.bcast[2];
}

// Ends a select over a short candidate set once at most kSmall candidates
// match the digits resolved so far (the keys of the bin holding the k-th
// largest; `remaining` of them, 1 <= remaining <= their count, belong to the
// top k), instead of the radix passes left: the keys of the bin are collected
// in LDS and wave 0 ranks them, one per lane, against each other. match(key)
// tells a key of the bin. Every lane must call it. (Measured on rows of at most
// 4096 positions: top-k 5.4 -> 5.0 us at 64 requests of 128 positions; the
// ranged select over longer rows' candidates ends this way once at most
// kSmallRanged keys remain.)
template <typename Match>
__device__ __forceinline__ void finish_small(const Slots& sl, uint32_t remaining, Match match, uint32_t& T, uint32_t& r) {
  const int tid = threadIdx.x;
  // (rs.small_n is zero from clear_hists: a select finishes this way once)
  for (int i = sl.first; i < sl.end; i += sl.step) {
    const uint32_t kk = rs.cand_key[sl.base + i];
    if (match(kk)) rs.small[atomicAdd(&rs.small_n, 1u)] = kk;  // exactly the bin's count, <= kSmall
  }
  __syncthreads();
  if ((tid >> 6) == 0) {
    const int m = __builtin_amdgcn_readfirstlane((int)rs.small_n);
    uint32_t mine, gt = 0u, ge = 0u;  // this lane's key; keys of the bin above / at or above it
    if (m <= 16) {
      // a few keys: every lane reads each key from the lane holding it
      mine = tid < m ? rs.small[tid] : 0u;
      for (int i = 0; i < m; ++i) {
        const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)mine, i);
        gt += v > mine ? 1u : 0u;
        ge += v >= mine ? 1u : 0u;
      }
    } else {
      // more keys: 16 at a time from broadcast LDS reads (a readlane per key
      // costs about 100 cycles: 2.5 us for 60 keys, against 0.35 us so; for
      // 16 keys or fewer the readlanes are the faster, by about 0.2 us on c3).
      // Slots past m hold key 0, below every key of the bin (wave 0's own
      // LDS stores are ordered before its loads).
      if (tid >= m) rs.small[tid] = 0u;
      mine = tid < m ? rs.small[tid] : 0u;
      for (int g = 0; 16 * g < m; ++g) {
        u32x4 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = *reinterpret_cast<const u32x4*>(&rs.small[16 * g + 4 * c]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            gt += v[c][e] > mine ? 1u : 0u;
            ge += v[c][e] >= mine ? 1u : 0u;
          }
      }
    }
    // the remaining-th largest: fewer than `remaining` keys above it, at least that many at or above
    const uint64_t hit = __ballot(tid < m && gt < remaining && ge >= remaining);
    const int src = hit ? __builtin_ctzll(hit) : 0;
    if (tid == 0) {
      rs.bcast[0] = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
      rs.bcast[1] = remaining - (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
    }
  }
  __syncthreads();
  T = rs.bcast[0];
  r = rs.bcast[1];
}

// Exact radix select over the n candidates in LDS (n >= k): the k-th largest
// key T and r, the number of keys == T taken. The histograms are clear on
// entry. With from_hist, the first digit (bin0) and the count of keys in
// higher bins (above0) are known already and the first pass is skipped.
struct Kth {
  uint32_t T, r;
};
__device__ __forceinline__ Kth select_candidates(const Slots& sl, int k, bool from_hist, uint32_t bin0, uint32_t above0) {
  uint32_t T = from_hist ? bin0 << 21 : 0u;
  uint32_t mask = from_hist ? 0xFFE00000u : 0u;
  uint32_t remaining = (uint32_t)k - (from_hist ? above0 : 0u);
  auto count = [&](uint32_t* h, int shift, uint32_t dmask) {
    int i = sl.first;
    for (; i + 3 * sl.step < sl.end; i += 4 * sl.step) {
      uint32_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kk[u] = rs.cand_key[sl.base + i + u * sl.step];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if ((kk[u] & mask) == T) atomicAdd(&h[hslot((kk[u] >> shift) & dmask)], 1u);
    }
    for (; i < sl.end; i += sl.step) {
      const uint32_t kk = rs.cand_key[sl.base + i];
      if ((kk & mask) == T) atomicAdd(&h[hslot((kk >> shift) & dmask)], 1u);
    }
  };
  auto in_bin = [&](uint32_t kk) { return (kk & mask) == T; };
  uint32_t r;
  if (!from_hist) {
    if (radix_pass<0>(T, mask, remaining, count) <= (uint32_t)kSmall) {
      finish_small(sl, remaining, in_bin, T, r);
      return Kth{T, r};
    }
  }
  if (radix_pass<1>(T, mask, remaining, count) <= (uint32_t)kSmall) {
    finish_small(sl, remaining, in_bin, T, r);
    return Kth{T, r};
  }
  radix_pass<2>(T, mask, remaining, count);
  return Kth{T, remaining};
}

// Exact radix select over the candidates in LDS at or above base, the
// largest segment cut. The candidates hold the whole top k exactly when its
// k-th largest key T is >= base, so keys below base never decide T: the
// digits (11, 11, then at most 10 bits) are those of the offset key - base,
// starting at the top bit of the range [base, largest key]. That range is
// narrow (the candidates above a cut share a few bins of the key's own first
// digit, where the first pass would pile its LDS atomics onto a few words).
// Returns r = 0xFFFFFFFF if fewer than k keys reach base (T < base: the caller
// selects over the whole row). Inline: as an out-of-line call it saved and
// restored 40 registers per lane through scratch memory on every call (c3
// top-k 14.56 -> 14.24 us inline). The histograms are clear on entry,
// and rs.range is (0, 0), or with preset every candidate is at or above base
// and rs.range[1] is the largest key.
__device__ __forceinline__ Kth select_candidates_ranged(const Slots& sl, int n, int k, uint32_t base, bool preset) {
  const int tid = threadIdx.x;
  uint32_t n_above = (uint32_t)n;
  if (!preset) {  // (else the gather left rs.range[1] set)
    uint32_t hi = 0u, above = 0u;
    for (int i = sl.first; i < sl.end; i += sl.step) {
      const uint32_t kk = rs.cand_key[sl.base + i];
      hi = max(hi, kk);
      above += kk >= base ? 1u : 0u;
    }
    hi = wave_max(hi);
    above = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(above), 63);
    if ((tid & 63) == 0) {
      atomicAdd(&rs.range[0], above);
      atomicMax(&rs.range[1], hi);
    }
    __syncthreads();
    n_above = rs.range[0];
  }
  if (n_above < (uint32_t)k) return Kth{0u, 0xFFFFFFFFu};
  const uint32_t span = rs.range[1] - base;
  int top = span == 0u ? 0 : 32 - __builtin_clz(span);  // bits of the offsets still to resolve
  uint32_t prefix = 0u, remaining = (uint32_t)k;
  for (int pass = 0; top > 0; ++pass) {  // at most three passes (11 + 11 + 10 bits)
    const int low = max(top - 11, 0), width = top - low;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* h = pass_hist(pass);
    // Four keys a lane per round, without branches: the reads may run past
    // the end (into cand_pos: n + 3 kRowThreads, and a region's end + 3 x 64,
    // stay below 2 kSlots), and a key not counted
    // adds to the lane's own dummy word instead of a bin. (The same sweep on
    // the first 4 or 8 waves only, the others passing the barrier: c3 top-k
    // 12.21 -> 13.13 / 12.49 us. With fewer waves the LDS latency shows.)
    for (int i = sl.first; i < sl.end; i += 4 * sl.step) {
      uint32_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) kk[u] = rs.cand_key[sl.base + i + u * sl.step];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t o = kk[u] - base;
        // o >> top in two shifts (top is 1 .. 32)
        const bool c = (i + u * sl.step < sl.end) & (kk[u] >= base) & (((o >> (top - 1)) >> 1) == prefix);
        const uint32_t bin = hslot((o >> low) & dmask);
        atomicAdd(c ? &h[bin] : &rs.dummy[tid & 63], 1u);
      }
    }
    __syncthreads();
    if (pass < 2) block_pick<kBins>(h, [&](uint32_t) { return remaining; });
    else block_pick<kBins / 2>(h, [&](uint32_t) { return remaining; });
    prefix = (prefix << width) | rs.bcast[0];
    remaining -= rs.bcast[1];
    top = low;
    const uint32_t in_bin = rs.bcast[2];
    // (bcast is written again only after the next pass's first barrier)
    if (top > 0 && in_bin <= (uint32_t)kSmallRanged) {
      uint32_t T, r;
      finish_small(sl, remaining, [&](uint32_t kk) {
        return kk >= base && (uint32_t)((uint64_t)(kk - base) >> top) == prefix; }, T, r);
      return Kth{T, r};
    }
  }
  return Kth{base + prefix, remaining};
}

// Writes the chosen positions from the n candidates in LDS (position order:
// with kReg, region after region in wave order, each in position order);
// each lane takes a run of consecutive candidates (of its wave's region).
__device__ __forceinline__ void write_from_candidates(const Slots& sl, Kth t, rsrc_t oi, rsrc_t ov, bool with_vals, bool raw) {
  const int m = sl.end, first = sl.first;  // candidates of the region (or the row), this lane's index among its lanes
  const int per = (m + sl.step - 1) / sl.step;  // <= kCap / kRowThreads, or kRegion / 64
  const int c0 = sl.base + min(first * per, m), c1 = sl.base + min(first * per + per, m);
  uint32_t n_gt = 0, n_eq = 0;
  for (int i = c0; i < c1; ++i) {
    const uint32_t kk = rs.cand_key[i];
    n_gt += kk > t.T ? 1u : 0u;
    n_eq += kk == t.T ? 1u : 0u;
  }
  const uint32_t my_gt = n_gt, my_eq = n_eq;
  uint32_t tot_gt, tot_eq;
  block_scan2(n_gt, n_eq, rs.part, &tot_gt, &tot_eq);
  uint32_t eq_rank = n_eq - my_eq;
  uint32_t pos = (n_gt - my_gt) + min(t.r, eq_rank);
  for (int i = c0; i < c1; ++i) {
    const uint32_t kk = rs.cand_key[i];
    if (kk > t.T || (kk == t.T && eq_rank < t.r)) {
      store_b32(oi, (int)pos, rs.cand_pos[i]);
      if (with_vals) store_b32(ov, (int)pos, raw ? kk : key_to_bits(kk));
      ++pos;
    }
    eq_rank += kk == t.T ? 1u : 0u;
  }
}

// Whole-row path: the same radix select over every key of the row, re-reading
// it from memory in every sweep. The histograms are clear on entry. Inline: as
// an out-of-line call it set every row kernel's register budget to the
// callee's (102 VGPRs, against 58-67 inline) and gave the kernels scratch
// memory for one saved register; inline, the 1M-token-width top-k took 6.08 ->
// 5.69 us, the other workloads within 0.05 us.
__device__ __forceinline__ void select_whole_row(rsrc_t row, int len, int k, rsrc_t oi, rsrc_t ov, bool with_vals) {
  const int tid = threadIdx.x;
  uint32_t T = 0u, mask = 0u, remaining = (uint32_t)k;
  auto count = [&](uint32_t* h, int shift, uint32_t dmask) {
    for (int i0 = 0; i0 < len; i0 += 8 * kRowThreads) {
      uint32_t kk[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) kk[u] = load_b32(row, i0 + u * kRowThreads + tid);  // 0 past len
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t x = i0 + u * kRowThreads + tid < len ? order_key(__uint_as_float(kk[u])) : 0u;
        if (x != 0u && (x & mask) == T) atomicAdd(&h[hslot((x >> shift) & dmask)], 1u);
      }
    }
  };
  radix_pass<0>(T, mask, remaining, count);
  radix_pass<1>(T, mask, remaining, count);
  radix_pass<2>(T, mask, remaining, count);
  uint32_t gt_seen = 0, eq_seen = 0;  // workgroup-uniform totals of earlier blocks
  for (int blk = 0; blk < len; blk += kSweep) {
    const int base = blk + 16 * tid;
    uint32_t key[16];
    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) key[j] = load_b32(row, base + j);  // 0 past len
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      key[j] = base + j < len ? order_key(__uint_as_float(key[j])) : 0u;
      n_gt += key[j] > T ? 1u : 0u;
      n_eq += key[j] == T ? 1u : 0u;
    }
    const uint32_t my_gt = n_gt, my_eq = n_eq;
    uint32_t tot_gt, tot_eq;
    block_scan2(n_gt, n_eq, rs.part, &tot_gt, &tot_eq);
    uint32_t eq_rank = eq_seen + n_eq - my_eq;
    uint32_t pos = gt_seen + (n_gt - my_gt) + min(remaining, eq_rank);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool gt = key[j] > T, eq = key[j] == T;
      if (gt || (eq && eq_rank < remaining)) {
        store_b32(oi, (int)pos, (uint32_t)(base + j));
        if (with_vals) store_b32(ov, (int)pos, key_to_bits(key[j]));
        ++pos;
      }
      eq_rank += eq ? 1u : 0u;
    }
    gt_seen += tot_gt;
    eq_seen += tot_eq;
  }
}

// Gathers the kept pairs of a row longer than kSeg into LDS, in sub-slot
// order; returns the candidate count, or -1 if more than kCap. Raises
// rs.max_cut (zero on entry) to the largest segment cut.
__device__ __forceinline__ int gather_segments(const uint32_t* __restrict__ ws, int b, int batch, int n_seg, int len) {
  const int tid = threadIdx.x;
  const int n_act = (len + kSeg - 1) / kSeg;
  const int n_sub = n_act * kSegWaves;
  const rsrc_t recs = make_rsrc(ws + (size_t)b * n_seg * kRecWords, (uint32_t)n_act * kRecWords * 4u);
  const rsrc_t pairs = make_rsrc(ws + ws_pairs(b, batch, n_seg), (uint32_t)n_act * kSeg * 8u);
  const int n_spec = min(kSpecSlots, n_sub);
  int n = 0;
  for (int c0 = 0; c0 < n_sub; c0 += kRound) {  // gather rounds of kRound sub-slots
    const int u = c0 + tid;
    const bool mine = tid < kRound && u < n_sub;
    uint32_t cnt = 0u, cut = 0u;
    if (mine) {
      const int s = u / kSegWaves;
      cnt = load_b32(recs, s * kRecWords + u % kSegWaves);
      cut = (u % kSegWaves == 0) ? load_b32(recs, s * kRecWords + kSegWaves) : 0u;
    }
    // read ahead (first round): pairs 2q, 2q + 1 of the first kSpecSlots
    // sub-slots' first kSpec pairs, q = tid + kRowThreads w
    u32x4 spec[4];
    if (c0 == 0) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int q = 2 * (tid + kRowThreads * w), v = q / kSpec, i = q % kSpec;
        if (v < n_spec) spec[w] = __builtin_amdgcn_raw_buffer_load_b128(pairs, (v * kSub + i) * 8, 0, 0);
      }
    }
    const uint32_t m = wave_max(cut);
    // pairs not read ahead
    const uint32_t rest = (u < n_spec) ? (cnt > (uint32_t)kSpec ? cnt - kSpec : 0u) : cnt;
    uint32_t incl = cnt, rincl = rest, tot, rtot;
    block_scan2(incl, rincl, rs.part, &tot, &rtot);  // (its barriers also order max_cut's clearing)
    if ((tid & 63) == 0) atomicMax(&rs.max_cut, m);
    if ((uint32_t)n + tot > (uint32_t)kCap) return -1;  // workgroup-uniform
    if (tid < kRound) {
      rs.cnt[tid] = cnt;
      rs.off[tid] = (uint32_t)n + incl - cnt;
      rs.roff[tid] = rincl - rest;
    }
    __syncthreads();
    if (c0 == 0) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int q = 2 * (tid + kRowThreads * w), v = q / kSpec, i = q % kSpec;
        if (v < n_spec) {
          const uint32_t cv = rs.cnt[v], ov = rs.off[v];
          if ((uint32_t)i < cv) {
            rs.cand_key[ov + i] = spec[w][0];
            rs.cand_pos[ov + i] = spec[w][1];
          }
          if ((uint32_t)i + 1 < cv) {
            rs.cand_key[ov + i + 1] = spec[w][2];
            rs.cand_pos[ov + i + 1] = spec[w][3];
          }
        }
      }
    }
    // the rest, as one list over the round's sub-slots
    const int m_sub = min(kRound, n_sub - c0);
    constexpr int kUnroll = 4;
    for (int j0 = 0; j0 < (int)rtot; j0 += kUnroll * kRowThreads) {
      int src[kUnroll], dst[kUnroll];
#pragma unroll
      for (int w = 0; w < kUnroll; ++w) {
        const int j = j0 + w * kRowThreads + tid;
        src[w] = 0;
        dst[w] = -1;
        if (j < (int)rtot) {
          // the sub-slot holding item j: the last one whose offset is <= j
          int lo = 0, hi = m_sub;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (rs.roff[mid] <= (uint32_t)j) lo = mid;
            else hi = mid;
          }
          const int skip = (c0 + lo < n_spec) ? kSpec : 0;
          const int i = skip + (j - (int)rs.roff[lo]);  // pair index within the sub-slot
          src[w] = (c0 + lo) * kSub + i;
          dst[w] = (int)rs.off[lo] + i;
        }
      }
      u32x2 c[kUnroll];
#pragma unroll
      for (int w = 0; w < kUnroll; ++w) c[w] = load_pair(pairs, src[w]);
#pragma unroll
      for (int w = 0; w < kUnroll; ++w) {
        if (dst[w] >= 0) {
          rs.cand_key[dst[w]] = c[w].x;
          rs.cand_pos[dst[w]] = c[w].y;
        }
      }
    }
    n += (int)tot;
    __syncthreads();  // cnt, off and roff are rewritten by the next round
  }
  return n;
}

// Inclusive scans of the kN values of every lane over the workgroup's lanes in
// lane order, and their totals. Every lane must call it; it ends with a
// barrier, after which rs.part may be rewritten.
template <int kN>
__device__ __forceinline__ void block_scan_n(uint32_t (&v)[kN], uint32_t (&tot)[kN]) {
  static_assert(kN <= 4, "rs.part holds four values per wave");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int q = 0; q < kN; ++q) v[q] = wave_inclusive_scan(v[q]);
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < kN; ++q) rs.part[4 * wave + q] = v[q];
  }
  __syncthreads();
  uint32_t before[kN];
  wave_partials<kN>(rs.part, before, tot);
#pragma unroll
  for (int q = 0; q < kN; ++q) v[q] += before[q];
  __syncthreads();
}

// The candidates of a row of kSeg < len <= kRes positions when the row width
// is at most kRes (no segment kernel ran): the workgroup loads the whole row
// into registers, each wave a contiguous chunk of it (C positions, a multiple
// of 64, at most 2048; lane l holds chunk positions 256 j + 64 e + l), cuts
// it, and each wave writes its keys at or above the cut with their positions
// to its own region of LDS, in position order, as they arrive: the regions
// in wave order are the candidates in position order. Returns the wave's
// count; adds it to rs.range[0] (kOverflow for a region that overflowed),
// which the caller reads after a barrier. Sets rs.max_cut to the cut, which
// the select and its check then treat as the largest segment cut: if the
// k-th largest key lies below it, the row takes the whole-row select, so the
// cut never changes the result, and rs.range[1] to the largest candidate
// key, which the ranged select would otherwise sweep the candidates for.
//
// The cut: with the score kernel's histogram (hint, and wave 0's pick of it
// in rs.hpick), that pick's bin edge. Otherwise a sample of n_s = kSamples
// keys, 64 runs of 32 consecutive positions (one 128-byte line each) spread
// evenly over the row and loaded by every wave before any of the row, so
// that the cut is picked while the row is still arriving, is counted into a
// first-digit histogram; the cut is the lower edge of the bin holding its
// rank_s-th largest, rank_s = 1.1 m + 4 sqrt(m) + 4 for m = k n_s / len the
// sample's expected share of the top k, and a bin holding more than 32
// samples is split by a second digit over the samples in it. (On the c3
// workload's rows longer than 4096: about 3000 candidates for k = 2048.) The
// sample histograms live in rs.cand_pos, which the candidates overwrite
// afterwards. The three radix histograms are untouched.
//
// Writing the candidates: for each of the 32 keys a lane holds (64
// consecutive positions across the wave), the wave takes a ballot of the
// kept ones and each kept key goes to the next free slot of the region in
// lane order, so no scan over the workgroup is needed and no barrier comes
// until all are stored, and a wave stores each block as it arrives. (Against
// 16-byte loads of four positions per lane spread over the row, a
// workgroup-wide scan of the kept counts and stores after the whole row had
// arrived: c3 top-k 11.8 -> 11.4 us, full 12.1 -> 11.7.) The values stored
// are the raw score bits; with a cut above +0 they stay so (raw is set: the
// select then works on raw bits, see below), otherwise each wave turns its
// own into keys.
__device__ __forceinline__ int gather_resident(const float* row_ptr, int len, int k, bool hint, bool& raw) {
  const int tid = threadIdx.x;
  // only positions [0, len) are readable through r1: a load reaching past
  // len reads 0 for each word past it (the range is checked per word)
  const rsrc_t r1 = make_rsrc(row_ptr, (uint32_t)len * 4u);
  // the sample first: 64 runs of 32 consecutive positions spread over the
  // row (two positions per lane), so the cut is picked while the row arrives
  const uint32_t run = (uint32_t)tid / 16u;
  const uint32_t run0 = min((run * (uint32_t)len / 64u) & ~31u, (uint32_t)len - 32u);
  const u32x2 sbits = __builtin_amdgcn_raw_buffer_load_b64(r1, (int)(run0 + 2u * ((uint32_t)tid & 15u)) * 4, 0, 0);
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  uint32_t* sample_hist = rs.cand_pos;  // two histograms of kBins
  *reinterpret_cast<u32x4*>(sample_hist + 4 * tid) = zero4;
  static_assert(4 * kRowThreads == 2 * kBins, "one 16-byte store per lane clears both");
  // (the barrier does not wait for loads: every wave's sample load is issued
  // before any row load, so the samples come back first)
  __syncthreads();
  // this wave's chunk of the row: c0 + [0, cl), C positions (a multiple of
  // 64, at most 2048) per wave; lane l holds positions c0 + 256 j + 64 e + l
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int C = (len + 64 * kRowWaves - 1) / (64 * kRowWaves) * 64;
  const int c0 = wave * C, cl = min(max(len - c0, 0), C), nb = (cl + 255) / 256;
  const rsrc_t rc = make_rsrc(row_ptr + min(c0, len), (uint32_t)cl * 4u);  // reads past cl return 0
  uint32_t v[kResBlk][4];
#pragma unroll
  for (int j = 0; j < kResBlk; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) v[j][e] = __builtin_amdgcn_raw_buffer_load_b32(rc, (256 * j + 64 * e + lane) * 4, 0, 0);

  uint32_t lo;
  const uint32_t n_s = kSamples;
  const float m = (float)k * (float)n_s / (float)len;
  const float want = 1.1f * m + 4.0f * sqrtf(m) + 4.0f;
  if (hint && rs.hpick[2] != 0u) {
    lo = max(rs.hpick[0] << 21, 1u);
  } else if (want >= (float)n_s) {
    lo = 1u;  // every valid key
  } else {
    const uint32_t rank_s = (uint32_t)want;  // 1 .. n_s - 1
    const uint32_t sk[2] = {order_key(__uint_as_float(sbits.x)), order_key(__uint_as_float(sbits.y))};
#pragma unroll
    for (int i = 0; i < 2; ++i) atomicAdd(&sample_hist[hslot(sk[i] >> 21)], 1u);
    __syncthreads();
    block_pick<kBins>(sample_hist, [&](uint32_t) { return rank_s; });  // the total is n_s
    const uint32_t b0 = rs.bcast[0], above = rs.bcast[1], in_bin = rs.bcast[2];
    lo = b0 << 21;
    if (in_bin > 32u) {
      uint32_t* h2 = sample_hist + kBins;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if ((sk[i] >> 21) == b0) atomicAdd(&h2[hslot((sk[i] >> 10) & 0x7FFu)], 1u);
      __syncthreads();
      block_pick<kBins>(h2, [&](uint32_t) { return rank_s - above; });
      lo |= rs.bcast[0] << 10;
    }
    lo = max(lo, 1u);
  }

  // key >= lo <=> score >= the float of lo, except for NaN (key 1). With lo
  // at or below -inf's key the test is score >= -inf, which leaves out NaN
  // scores: they are the smallest keys, so they belong to the top k only if
  // fewer than k other keys are valid, and then the candidates fall short of
  // k and the whole-row select runs. Positions past the chunk (read as 0) of
  // its last block are set to a negative NaN first, so they fail the test
  // and stay below the raw-bits maximum.
  const float f = lo <= 0x007FFFFFu ? -__builtin_inff() : __uint_as_float(key_to_bits(lo));
  raw = !hint && lo > 0x80000000u;  // workgroup-uniform
  char* const reg = reinterpret_cast<char*>(rs.cand_key + wave * kRegion);  // rs.cand_pos lies kSlots words further
  uint32_t wo = 0u;  // the region's next free slot (wave-uniform)
  bool over = false;
  int im = 0;
#pragma unroll
  for (int j = 0; j < kResBlk; ++j) {
    if (j < nb && !over) {
      if (256 * (j + 1) > cl) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][e] = 256 * j + 64 * e + lane < cl ? v[j][e] : 0xFFC00000u;
      }
      // (raw: the largest held bits as signed integers, the largest score;
      // negative scores and the NaN set above are negative)
      if (raw) {
#pragma unroll
        for (int e = 0; e < 4; ++e) im = max(im, (int)v[j][e]);
      }
      bool c[4];
      uint64_t m[4];
      uint32_t cnt = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = __uint_as_float(v[j][e]) >= f;
        m[e] = __builtin_amdgcn_ballot_w64(c[e]);
        cnt += (uint32_t)__builtin_popcountll(m[e]);
      }
      over = wo + cnt > (uint32_t)kRegion;  // the row then takes the whole-row select
      if (!over) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (c[e]) {
            const uint32_t r =
                __builtin_amdgcn_mbcnt_hi((uint32_t)(m[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[e], 0u));
            uint32_t* const at = reinterpret_cast<uint32_t*>(reg + 4u * wo + 4u * r);
            at[0] = v[j][e];
            at[kSlots] = (uint32_t)(c0 + lane + 256 * j + 64 * e);  // rs.cand_pos
          }
          wo += (uint32_t)__builtin_popcountll(m[e]);
        }
      }
    }
  }
  // the largest candidate (A cut above +0 keeps only positive floats and
  // +inf, whose raw bits are ordered as their keys are, and differ from them
  // by the top bit only: the candidates then stay raw bits, and the select
  // and its check run on raw bits; the largest score bounds them);
  // otherwise the region's keys, turned into keys here
  const int nw = over ? 0 : (int)wo;
  uint32_t mx = (uint32_t)im;
  if (!raw) {
    uint32_t* const rk = reinterpret_cast<uint32_t*>(reg);
    mx = 0u;
    for (int i = lane; i < nw; i += 64) {
      const uint32_t kk = order_key(__uint_as_float(rk[i]));
      rk[i] = kk;
      mx = max(mx, kk);
    }
  }
  mx = wave_max(mx);
  if (lane == 0) {
    atomicAdd(&rs.range[0], over ? kOverflow : wo);
    atomicMax(&rs.range[1], mx);
  }
  if (tid == 0) rs.max_cut = raw ? (lo & 0x7FFFFFFFu) : lo;
  return nw;
}

// A row of at most kSeg positions in the regions' layout: lane t loads
// positions 4t .. 4t + 3, and wave w's region holds the valid positions
// 256 w + i at slot i, as keys. Returns the wave's count; every valid key is
// a candidate, so the row's is len.
__device__ __forceinline__ int load_short_regions(const float* row_ptr, int len) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(row_ptr, (uint32_t)len * 4u), 16 * tid, 0, 0);
  uint32_t* const rk = rs.cand_key + wave * kRegion;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int p = 4 * tid + e;
    if (p < len) {
      rk[4 * lane + e] = order_key(__uint_as_float(x[e]));
      rk[4 * lane + e + kSlots] = (uint32_t)p;  // rs.cand_pos
    }
  }
  return min(max(len - 256 * wave, 0), 256);
}

// After a barrier: the candidates of all regions (rs.range[0]), or -1 if a
// region overflowed.
__device__ __forceinline__ int region_total() {
  const uint32_t t = rs.range[0];
  return t >= kOverflow ? -1 : (int)t;
}

// kWidth: the row width class, kNarrow (at most kSeg: every row is its own
// candidate set), kResident (at most kRes: rows held in registers) or kWide
// (the segment kernel ran); kHist: the score kernel's histogram is given.
// Compiled apart, so that each launch runs code holding only its own paths:
// the instruction cache is cold after a score launch (measured against one
// kernel for all: top-k c3 12.2 -> 11.8 us, full 12.5 -> 12.1, c2 5.7 ->
// 5.25, 64 rows of 128 positions 4.6 -> 4.2, the same at a 1M-token row
// width 6.5 -> 6.1).
enum { kNarrow = 0, kResident = 1, kWide = 2 };
template <int kWidth, bool kHist>
__global__ __launch_bounds__(kRowThreads) void topk_row_kernel(const float* __restrict__ logits,
                                                                const int32_t* __restrict__ seq_lens,
                                                                int32_t max_c4, int32_t k,
                                                                int32_t* __restrict__ out_idx,
                                                                float* __restrict__ out_vals,
                                                                const uint32_t* __restrict__ ws, int32_t n_seg,
                                                                uint32_t* __restrict__ hist) {
  const int b = blockIdx.x, tid = threadIdx.x;
  // this row's histogram, set back to zero for the next score call once read
  const rsrc_t hrow = make_rsrc(kHist ? hist + (size_t)b * kHistBins : nullptr, kHist ? kHistBins * 4u : 0u);
  static_assert(kHistBins == 2 * kRowThreads, "two bins per lane");
  auto clear_hist_row = [&]() { store_pair(hrow, tid, 0u, 0u); };
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
    if (kHist) clear_hist_row();
    for (int i = tid; i < k; i += kRowThreads) {
      store_b32(oi, i, i < len ? (uint32_t)i : 0xFFFFFFFFu);
      if (with_vals) store_b32(ov, i, i < len ? load_b32(row, i) : 0x7FC00000u);
    }
    return;
  }

  if (kHist && tid < 64) {
    const Pick p = pick_row_hist(load_row_hist(hist, b), k);
    if (tid == 0) {
      rs.hpick[0] = p.bin;
      rs.hpick[1] = p.above;
      rs.hpick[2] = p.ok ? 1u : 0u;
    }
  }
  clear_hists();
  // the resident kernel keeps its candidates in per-wave regions
  constexpr bool kReg = kWidth == kResident;
  int n;
  int nw = 0;  // kReg: this wave's candidates
  bool raw = false;  // candidates held as raw score bits (gather_resident)
  if (len <= kSeg) {
    // the row is its own candidate set
    if constexpr (kReg) {
      nw = load_short_regions(row_ptr, len);
    } else {
      uint32_t bits[kSeg / kRowThreads];
#pragma unroll
      for (int m = 0; m < kSeg / kRowThreads; ++m) bits[m] = load_b32(row, m * kRowThreads + tid);  // 0 past len
#pragma unroll
      for (int m = 0; m < kSeg / kRowThreads; ++m) {
        const int i = m * kRowThreads + tid;
        if (i < len) {
          rs.cand_key[i] = order_key(__uint_as_float(bits[m]));
          rs.cand_pos[i] = (uint32_t)i;
        }
      }
      n = len;
    }
  } else if constexpr (kWidth == kResident) {
    nw = gather_resident(row_ptr, len, k, kHist, raw);
  } else if constexpr (kWidth == kWide) {
    n = gather_segments(ws, b, (int)gridDim.x, n_seg, len);
  }
  __syncthreads();
  if constexpr (kReg) n = len <= kSeg ? len : region_total();
  const Slots sl = kReg ? region_slots(nw) : all_slots(n);
  bool from_hist = kHist && rs.hpick[2] != 0u;
  uint32_t bin0 = 0u, above0 = 0u;
  if (kHist) clear_hist_row();  // wave 0 read it before the barrier
  if (from_hist && n >= k) {
    // The histogram is taken only where the candidates confirm it: fewer than
    // k of them above its bin and at least k in or above it. The candidates
    // hold every key at or above the bin's lower edge (each segment cut there;
    // a short row is all candidates), so these counts are exact, and the
    // count above comes from them: counts that do not belong to these logits
    // cannot change the result.
    bin0 = rs.hpick[0];
    uint32_t ab = 0u, ge = 0u, tot_ab, tot_ge;
    for (int i = sl.first; i < sl.end; i += sl.step) {
      const uint32_t d = rs.cand_key[sl.base + i] >> 21;
      ab += d > bin0 ? 1u : 0u;
      ge += d >= bin0 ? 1u : 0u;
    }
    block_scan2(ab, ge, rs.part, &tot_ab, &tot_ge);
    from_hist = tot_ab < (uint32_t)k && tot_ge >= (uint32_t)k;
    above0 = tot_ab;
  }
  if (n >= k) {  // n < 0: more than kCap candidates
    // gathered candidates: the select over those at or above the largest cut
    // (with a histogram that the candidates did not confirm, the ranged select
    // over the candidates at or above the largest cut decides, as without one)
    Kth t;
    if constexpr (kWidth == kNarrow) {
      t = select_candidates(sl, k, from_hist, bin0, above0);
    } else {
      t = (!from_hist && len > kSeg) ? select_candidates_ranged(sl, n, k, rs.max_cut, kReg)
                                     : select_candidates(sl, k, from_hist, bin0, above0);
    }
    // every key a segment left out lies below its cut, hence below T
    if (t.r != 0xFFFFFFFFu && t.T >= rs.max_cut) {
      write_from_candidates(sl, t, oi, ov, with_vals, raw);
      return;
    }
    __syncthreads();  // every wave is done with the histograms
    clear_hists();
    __syncthreads();
  }
  select_whole_row(row, len, k, oi, ov, with_vals);
}

}  // namespace

size_t topk_workspace_words(int32_t batch, int32_t max_c4) {
  if (max_c4 <= kRes) return 0;  // no segment kernel
  const size_t n_seg = ((size_t)max_c4 + kSeg - 1) / kSeg;
  return (size_t)batch * n_seg * (kRecWords + 2 * kSeg);  // records, then pairs
}

hipError_t launch_topk(const float* logits, const int32_t* seq_lens, int32_t batch, int32_t max_c4,
                       int32_t k, int32_t* out_idx, float* out_vals, void* workspace, uint32_t* hist,
                       hipStream_t stream) {
  const int n_seg = (int)(((int64_t)max_c4 + kSeg - 1) / kSeg);
  uint32_t* ws = static_cast<uint32_t*>(workspace);
  // a row reaches the segment kernel only if it is longer than kSeg and than
  // k, and only where the row width exceeds kRes
  if (max_c4 > kRes && k < max_c4)
    hipLaunchKernelGGL(topk_segment_kernel, dim3(batch, min(n_seg, kSegGridY)), dim3(kSegThreads), 0, stream, logits, seq_lens,
                       max_c4, k, n_seg, ws, hist);
  const int width = max_c4 <= kSeg ? kNarrow : (max_c4 <= kRes ? kResident : kWide);
#define DSA_ROW_LAUNCH(W, H)                                                                                   \
  hipLaunchKernelGGL((topk_row_kernel<W, H>), dim3(batch), dim3(kRowThreads), 0, stream, logits, seq_lens, max_c4, \
                     k, out_idx, out_vals, ws, n_seg, hist)
  if (hist == nullptr) {
    if (width == kNarrow) DSA_ROW_LAUNCH(kNarrow, false);
    else if (width == kResident) DSA_ROW_LAUNCH(kResident, false);
    else DSA_ROW_LAUNCH(kWide, false);
  } else {
    if (width == kNarrow) DSA_ROW_LAUNCH(kNarrow, true);
    else if (width == kResident) DSA_ROW_LAUNCH(kResident, true);
    else DSA_ROW_LAUNCH(kWide, true);
  }
#undef DSA_ROW_LAUNCH
  return hipGetLastError();
}

}  // namespace dsa
