// Score kernel of the DSA indexer decode step on gfx950.
//
// What it computes (page "The O(Actual) Indexer", section "The Bottleneck That
// Was"; page "The Moment of Breakthrough", section "The Context"): for request
// b and every c4 position s below its length,
//     logits[b][s] = sum_h w[b][h] * max(0, q[b][h] . k[page_table[b][s/64]][s%64])
// and -inf at every position at or past the length, over a row of
// max_pages * 64 positions.
//
// Work lists. The work of one call is two flat lists: every valid page of
// every request (request-major, page-minor), and the -inf tails. In the
// stateless mode the tail of a request runs from its first page past the
// length to the row end, cut into chunks of kTailChunk positions. In the
// incremental mode each request's tail is one item: the wave that takes it
// reads the request's previous high-water mark, rewrites -inf only up to the
// page holding it (everything beyond is -inf already) and then stores the new
// mark; no other wave reads that mark, so the update needs no second kernel.
// A fixed grid of one-wave workgroups, as
// many as the chip keeps resident (capped by the largest list the shapes
// allow), splits each list into equal contiguous ranges when every
// workgroup gets pages (a workgroup scores its pages, then writes its tail
// chunks: writes between the page reads slow the read stream), and splits the
// two lists as one otherwise (the workgroups past the pages take the tail).
// The grid holds eight workgroups per compute unit. The launch shape
// depends only on (batch, max_pages), so it can be captured once and replayed
// for any lengths, and the work and HBM traffic follow the actual lengths:
// pages past a length are never read (the early exit of the section "The
// Benchmark Results"), and in the incremental mode the tail is not rewritten.
// Each workgroup finds the requests its range starts in with wave scans over
// windows of 64 request lengths, walks its range in order, and loads q and w
// only when the request changes. The walk is a three-stage pipeline: while a
// page is computed, the next page's keys and the page id after it are in
// flight.
//
// A page is read with eight fully coalesced 1 KiB wave loads, staged in LDS
// under an XOR swizzle, and contracted against the request's 32 x 64 query
// block with eight v_mfma_f32_32x32x16_bf16 (bf16 products, fp32
// accumulation). The accumulator holds the 32 heads x 32 positions of each
// half page with one position per lane; ReLU, the head weights and 16 of the
// 32 heads are summed in registers, and one cross-half lane exchange
// (v_permlane32_swap) adds the other 16 heads. The tail is written with
// 16-byte stores, 1 KiB per wave instruction.
//
// fp8 keys (score_kernel<true>): a page is 4 KiB of OCP FP8 E4M3 codes plus
// one float32 scale per key. The codes are staged in LDS under an XOR swizzle
// of 8-byte chunks and converted to bfloat16 as the MFMA operand is read (the
// conversion is exact: every e4m3 value is a bfloat16 value); the dot
// products are then multiplied by their key's scale before the ReLU, which is
// the formula on the scaled key.
//
// Several query tokens (score_kernel<false, kTok>, kTok = 2..4: the current
// token and draft tokens, each with its own causal length): a page is staged
// once and contracted against each token's query block; the work list covers
// the pages below the longest of a request's lengths, and each token's row is
// masked at its own length. Logits are [batch][kTok][width] and the tail is
// written for every token row (the stateless mode).
#include "common.h"

namespace dsa {
namespace {

constexpr int kTailChunk = 4096;  // positions per tail item (16 KiB of -inf)

__device__ __forceinline__ int clamp_len(int len, int width) { return min(max(len, 0), width); }

// LDS slot of 16-byte chunk `col` (0..7) of key row `row` (0..63). Each key row
// is 128 B; XOR-ing the chunk index with the row keeps the eight rows read by
// consecutive lanes of an MFMA operand load on distinct banks.
__device__ __forceinline__ int lds_slot(int row, int col) { return row * 8 + (col ^ (row & 7)); }

// Inclusive scan over the 64 lanes of a wave (row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_total(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(v), 63);
}

struct Shape {
  rsrc_t lens;   // int32 [batch][tok]
  rsrc_t marks;  // int32 [batch] high-water marks, if `incremental` (tok == 1 only)
  bool incremental;
  int batch, width, tok;
};

// Request b's share of the work: its valid pages (those below the longest of
// its tokens' lengths, len), and its -inf tail from position tail0: chunks of
// kTailChunk up to the row end (stateless mode), or one item (incremental
// mode). Reads the lengths only, never the marks.
struct RowWork {
  uint32_t pages, chunks, tail0, len;
};
__device__ __forceinline__ RowWork row_work(const Shape& sh, int b) {
  RowWork r{0, 0, 0, 0};
  if (b < sh.batch) {
    int len = 0;
    for (int t = 0; t < sh.tok; ++t)
      len = max(len, clamp_len((int)__builtin_amdgcn_raw_buffer_load_b32(sh.lens, (b * sh.tok + t) * 4, 0, 0), sh.width));
    r.len = (uint32_t)len;
    r.pages = (uint32_t)((len + kPage - 1) / kPage);
    r.tail0 = r.pages * kPage;
    r.chunks = sh.incremental ? 1u : ((uint32_t)sh.width - r.tail0 + kTailChunk - 1) / kTailChunk;
  }
  return r;
}

// A window of 64 requests over one of the two lists (pages or tail chunks):
// this lane's request count, its exclusive prefix inside the window, the
// window total, and the items before the window.
struct Window {
  int b0;
  uint32_t cnt, pre, tot, acc;
};
__device__ __forceinline__ void window_set(Window& W, const RowWork& r, bool tail) {
  W.cnt = tail ? r.chunks : r.pages;
  const uint32_t incl = wave_inclusive_scan(W.cnt);
  W.pre = incl - W.cnt;
  W.tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}
__device__ __forceinline__ void window_load(Window& W, const Shape& sh, bool tail) {
  window_set(W, row_work(sh, W.b0 + (int)(threadIdx.x & 63)), tail);
}
// Moves W forward to the window holding `item` (an index into its list, below
// the list total) and returns the request and the index inside the request.
__device__ __forceinline__ void window_find(Window& W, uint32_t item, const Shape& sh, bool tail, int& b,
                                            uint32_t& j) {
  while (item >= W.acc + W.tot && W.b0 + 64 < sh.batch) {
    W.acc += W.tot;
    W.b0 += 64;
    window_load(W, sh, tail);
  }
  const uint32_t r = item - W.acc;
  const uint64_t m = __ballot(W.cnt > 0 && W.pre + W.cnt > r);
  const int l = m ? __builtin_ctzll(m) : 0;  // never empty for an item below the list total
  b = min(W.b0 + l, sh.batch - 1);
  j = r - (uint32_t)__builtin_amdgcn_readlane((int)W.pre, l);
}

// Key page format: bfloat16 (8 KiB per page) or fp8 e4m3fn codes (4 KiB)
// with one float32 scale per key.
template <bool kFp8>
struct KeyFormat {
  static constexpr int kBytes = kFp8 ? kPageBytes / 2 : kPageBytes;  // key bytes per page
  static constexpr int kLoads = kBytes / 1024;                        // 16-byte loads per lane
};
// One page in flight: its key chunks and (fp8) the scales of this lane's two keys.
template <bool kFp8>
struct PageRegs {
  u32x4 v[KeyFormat<kFp8>::kLoads];
  float s0, s1;
};

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 8 e4m3fn codes (bytes of x, lowest first) -> 8 bfloat16 (exact)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(u32x2 x) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

// LDS 8-byte slot of chunk `j` (0..7, 8 dims each) of fp8 key row `row`:
// XOR-ing the chunk with the row keeps the rows read by consecutive lanes on
// distinct banks.
__device__ __forceinline__ int lds_slot8(int row, int j) { return row * 8 + (j ^ (row & 7)); }

// kTok query tokens per request (1: a plain decode step; more: the current
// token and draft tokens, each with its own causal length), every key page
// read once for all of them. Two resident waves per SIMD, measured against
// three: fewer, longer ranges write their logits in fewer, larger bursts,
// which slow the read stream less (bf16 keys: c3 -1.0 us, full -1.1 us; fp8
// keys: c3 -0.6 us, full -1.2 us).
template <bool kFp8, int kTok>
constexpr int waves_per_simd() { return 2; }

template <bool kFp8, int kTok>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(waves_per_simd<kFp8, kTok>(), waves_per_simd<kFp8, kTok>())))
void score_kernel(
    const uint16_t* __restrict__ q,          // bf16 [B][kTok][32][64]
    const float* __restrict__ w,             // [B][kTok][32]
    const void* __restrict__ k_pool,         // bf16 [num_pages][64][64], or e4m3fn codes [num_pages][64][64]
    const float* __restrict__ k_scale,       // fp8 only: [num_pages][64]
    int64_t num_pages,
    const int32_t* __restrict__ page_table,  // [B][max_pages]
    const int32_t* __restrict__ seq_lens,    // [B][kTok]
    int32_t batch, int32_t max_pages,
    float* __restrict__ logits,              // [B][kTok][max_pages * 64]
    int32_t* __restrict__ row_hwm,           // [B] or null: the longest of each request's token lengths
    uint32_t* __restrict__ hist)             // [B][kHistBins] or null (kTok == 1 only)
{
  const int lane = threadIdx.x;
  const int half = lane >> 5;
  const int n = lane & 31;
  // (the marks' resource is built from row_hwm alone, empty without it: were
  // it able to point at seq_lens, the stores of the new marks would keep the
  // compiler from reading the lengths through scalar loads, and the vector
  // loads it would use instead wait for every page load in flight)
  const Shape sh{make_rsrc(seq_lens, (uint32_t)(batch * kTok) * 4u),
                 make_rsrc(row_hwm, row_hwm != nullptr ? (uint32_t)batch * 4u : 0u),
                 row_hwm != nullptr, batch, max_pages * kPage, kTok};

  // list totals, then this workgroup's contiguous ranges: pages [s, pe) and
  // tail chunks [ts, te)
  uint32_t n_pages = 0, n_chunks = 0;
  RowWork first{0, 0, 0, 0};  // the first window's requests, kept: no second round trip for them
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const RowWork r = row_work(sh, b0 + lane);
    if (b0 == 0) first = r;
    n_pages += wave_total(r.pages);
    n_chunks += wave_total(r.chunks);
  }
  uint32_t s, pe, ts, te;
  if (n_pages >= gridDim.x) {
    // every workgroup has pages: each list split on its own, tail after pages
    const uint32_t per_p = (n_pages + gridDim.x - 1) / gridDim.x;
    s = min(n_pages, blockIdx.x * per_p);
    pe = min(n_pages, s + per_p);
    const uint32_t per_t = (n_chunks + gridDim.x - 1) / gridDim.x;
    ts = min(n_chunks, blockIdx.x * per_t);
    te = min(n_chunks, ts + per_t);
  } else {
    // fewer pages than workgroups: one list, pages then tail chunks, so that
    // the workgroups without pages take the tail
    const uint32_t total = n_pages + n_chunks, per = (total + gridDim.x - 1) / gridDim.x;
    const uint32_t a = min(total, blockIdx.x * per), z = min(total, a + per);
    s = min(a, n_pages);
    pe = min(z, n_pages);
    ts = max(a, n_pages) - n_pages;
    te = max(z, n_pages) - n_pages;
  }
  if (s >= pe && ts >= te) return;

  using Fmt = KeyFormat<kFp8>;
  using Regs = PageRegs<kFp8>;
  __shared__ u32x4 tile[kPageChunks];  // one bf16 page, or the first half for fp8

  // bf16 keys: a page's 64 scores (per query token) go to an LDS stash,
  // written out as runs of contiguous logits at the end of the workgroup's
  // pages (or when the stash is full) with 1 KiB wave stores.
  // Measured with a load probe over random 8 KiB pages: 256 B of results
  // stored after every page cost the read stream 6 us of 48 at 32768 pages;
  // the same bytes written in one burst per workgroup cost 2. (Measured in
  // the kernel: full 50.2 -> 48.4 us; two and three query tokens 1-2 us per
  // step faster; fp8 pages and four query tokens no gain, so they store per
  // page.) Every logits store is written through the L2 (kWriteThrough):
  // measured against streaming stores, the kernel alone is 0.3-0.4 us
  // slower, but a score and top-k step is 0.5-0.7 us faster (B = 64 at 128K
  // tokens; 0.3 us at B = 16 and 8K), since the kernel's end no longer
  // writes the logits back from the L2s before the top-k can start.
  constexpr bool kStashed = !kFp8 && kTok <= 3;
  constexpr int kStash = kTok == 1 ? 32 : 8;  // pages; token t's rows at [t][page][64]
  __shared__ __attribute__((aligned(16))) uint32_t stash[kStashed ? kTok * kStash * kPage : 4];
  __shared__ int stash_b[kStash], stash_j[kStash];
  int stash_n = 0;
  auto stash_flush = [&]() {
    __syncthreads();  // the stash writes are done
    int p = 0;
    while (p < stash_n) {
      // a run of consecutive pages of one request: contiguous logits
      const int rb = __builtin_amdgcn_readfirstlane(stash_b[p]);
      const int rj = __builtin_amdgcn_readfirstlane(stash_j[p]);
      int q = p + 1;
      while (q < stash_n && stash_b[q] == rb && stash_j[q] == rj + (q - p)) ++q;
      q = __builtin_amdgcn_readfirstlane(q);
      const int words = (q - p) * kPage;
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        const rsrc_t out = make_rsrc(logits + ((int64_t)rb * kTok + t) * sh.width + (int64_t)rj * kPage,
                                     (uint32_t)words * 4u);
        for (int w0 = lane * 4; w0 < words; w0 += 256)
          __builtin_amdgcn_raw_buffer_store_b128(
              *reinterpret_cast<const u32x4*>(&stash[(t * kStash + p) * kPage + w0]), out, w0 * 4, 0, kWriteThrough);
      }
      p = q;
    }
    __syncthreads();  // the stash is rewritten next
    stash_n = 0;
  };

  if (s < pe) {
    Window W{0, 0, 0, 0, 0};
    window_set(W, first, false);

    // Three-stage pipeline over the range: while item `it` is computed, the
    // key page of item it + 1 and the page id of item it + 2 are in flight.
    // Page ids come in through vector loads, so that all three kinds of load
    // complete in issue order and no wait for one stalls behind another; the
    // loop is unrolled twice with ping-pong registers, so no register holding
    // a pending load is ever copied (a copy would wait for the load). Every
    // step issues the same loads whatever the data (an item past the range or
    // an id outside the pool reads through an empty resource, which returns
    // zeros without a memory access), so the compiler's in-order wait counts
    // never fall back to waiting for everything in flight.
    const rsrc_t none = make_rsrc(k_pool, 0u);
    const char* const kbase = static_cast<const char*>(k_pool);
    // page id load of item x (pending until key_load reads it); `in` tells
    // whether x lies in the range (past it the load reads an empty resource)
    auto id_load = [&](uint32_t x, int& bx, uint32_t& jx, bool& in) -> uint32_t {
      in = x < pe;
      if (in) window_find(W, x, sh, false, bx, jx);
      const rsrc_t pt = in ? make_rsrc(page_table + (int64_t)bx * max_pages, (uint32_t)max_pages * 4u) : none;
      return __builtin_amdgcn_raw_buffer_load_b32(pt, in ? (int)jx * 4 : 0, 0, 0);
    };
    // key page of a loaded id into dst; false if the item is past the range
    // or the id is outside the pool (then dst is zero and no page is read)
    auto key_load = [&](uint32_t id, bool in, Regs& dst) -> bool {
      const int page = __builtin_amdgcn_readfirstlane((int)id);
      const bool ok = in && page >= 0 && (int64_t)page < num_pages;
      const rsrc_t kp = ok ? make_rsrc(kbase + (int64_t)page * Fmt::kBytes, Fmt::kBytes) : none;
      // 16-byte chunk c = 64 * i + lane of the page
#pragma unroll
      for (int i = 0; i < Fmt::kLoads; ++i)
        dst.v[i] = __builtin_amdgcn_raw_buffer_load_b128(kp, (i * 64 + lane) * 16, 0, kNonTemporal);
      if constexpr (kFp8) {
        // scales of this lane's keys n and n + 32
        const rsrc_t sp = ok ? make_rsrc(k_scale + (int64_t)page * kPage, kPage * 4u) : none;
        dst.s0 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sp, n * 4, 0, 0));
        dst.s1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sp, (n + 32) * 4, 0, 0));
      }
      return ok;
    };

    int q_row = -1;
    bf16x8 a[kTok][4];
    f32x4 wv[kTok][4];
    // q and w of request bx, if not held already; called before the phase's
    // other loads, so that waiting for them never waits for those
    auto ensure_qw = [&](int bx) {
      if (bx != q_row) {
        // query operand A (32 heads x 16 dims per step): lane holds head n,
        // dims 16*kb + 8*half .. +7 = chunk 2*kb + half of that head's row
        const rsrc_t qr = make_rsrc(q + (int64_t)bx * (kTok * kHeads * kDim), kTok * kHeads * kRowBytes);
#pragma unroll
        for (int t = 0; t < kTok; ++t)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            a[t][kb] = __builtin_bit_cast(
                bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            qr, (t * kHeads + n) * kRowBytes + (2 * kb + half) * 16, 0, 0));
        // head weights in accumulator order: register r of a lane holds head
        // 8*(r/4) + 4*half + r%4, so group g = r/4 is the float4 at head 8*g + 4*half
        const rsrc_t wr = make_rsrc(w + (int64_t)bx * kTok * kHeads, kTok * kHeads * sizeof(float));
#pragma unroll
        for (int t = 0; t < kTok; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            wv[t][g] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, (t * kHeads + 8 * g + 4 * half) * 4, 0, 0));
        q_row = bx;
      }
    };
    // scores of item (bx, jx) from its key page (q and w of bx held), for
    // each of the request's tokens
    auto compute = [&](int bx, uint32_t jx, bool okx, const Regs& page) {
      const int base = (int)jx * kPage;
      float val[kTok];
#pragma unroll
      for (int t = 0; t < kTok; ++t) val[t] = __builtin_nanf("");  // a page id outside the pool scores NaN
      if (okx) {
        // keys operand B (16 dims x 32 positions per step): lane holds position
        // n of each half page, dims 16*kb + 8*half .. +7
        bf16x8 b0[4], b1[4];
        if constexpr (!kFp8) {
          // 16-byte chunk c = 64 * i + lane is key row c / 8, column c % 8
#pragma unroll
          for (int i = 0; i < Fmt::kLoads; ++i) tile[lds_slot(i * 8 + (lane >> 3), lane & 7)] = page.v[i];
          __syncthreads();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int col = 2 * kb + half;
            b0[kb] = __builtin_bit_cast(bf16x8, tile[lds_slot(n, col)]);
            b1[kb] = __builtin_bit_cast(bf16x8, tile[lds_slot(n + 32, col)]);
          }
        } else {
          // 16-byte chunk c = 64 * i + lane is key row c / 4, dims 16 * (c % 4) .. +15:
          // two 8-byte chunks, stored at their swizzled slots
          u32x2* tile8 = reinterpret_cast<u32x2*>(tile);
#pragma unroll
          for (int i = 0; i < Fmt::kLoads; ++i) {
            const int c = i * 64 + lane, row = c >> 2, j = 2 * (c & 3);
            u32x2 lo, hi;
            lo[0] = page.v[i][0];
            lo[1] = page.v[i][1];
            hi[0] = page.v[i][2];
            hi[1] = page.v[i][3];
            tile8[lds_slot8(row, j)] = lo;
            tile8[lds_slot8(row, j + 1)] = hi;
          }
          __syncthreads();
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const int j = 2 * kb + half;
            b0[kb] = e4m3x8_to_bf16(tile8[lds_slot8(n, j)]);
            b1[kb] = e4m3x8_to_bf16(tile8[lds_slot8(n + 32, j)]);
          }
        }
        __syncthreads();  // the tile is rewritten for the next page
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
          f32x16 acc0 = {};  // positions 0..31 of the page
          f32x16 acc1 = {};  // positions 32..63
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kb], b0[kb], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][kb], b1[kb], acc1, 0, 0, 0);
          }
          if constexpr (kFp8) {
            // each dot product times its key's scale (this lane's keys n and n + 32)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc0[r] *= page.s0;
              acc1[r] *= page.s1;
            }
          }
          // weighted ReLU over this lane's 16 heads, then the other 16 from lane ^ 32
          float p0 = 0.f, p1 = 0.f;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              p0 = __builtin_fmaf(wv[t][g][r], __builtin_fmaxf(acc0[4 * g + r], 0.f), p0);
              p1 = __builtin_fmaf(wv[t][g][r], __builtin_fmaxf(acc1[4 * g + r], 0.f), p1);
            }
          }
          // lane < 32 owns position lane of the first half, lane >= 32 position lane of the second;
          // the other 16 heads of a position sit in lane ^ 32: one v_permlane32_swap hands p0's upper
          // half to the lower lanes and p1's lower half to the upper lanes
          const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, p0),
                                                           __builtin_bit_cast(uint32_t, p1), false, false);
          val[t] = half ? p1 + __builtin_bit_cast(float, (uint32_t)sw[0]) : p0 + __builtin_bit_cast(float, (uint32_t)sw[1]);
        }
      }
      if constexpr (kStashed) {
        if (stash_n == kStash) stash_flush();
        if (lane == 0) {
          stash_b[stash_n] = bx;
          stash_j[stash_n] = (int)jx;
        }
      }
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        const int len = clamp_len(seq_lens[bx * kTok + t], sh.width);
        const float v = base + lane >= len ? -__builtin_inff() : val[t];  // partial last page, shorter tokens
        if constexpr (kStashed) {
          stash[(t * kStash + stash_n) * kPage + lane] = __builtin_bit_cast(uint32_t, v);
        } else {
          const rsrc_t out = make_rsrc(logits + ((int64_t)bx * kTok + t) * sh.width + base, kPage * sizeof(float));
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), out, lane * 4, 0, kWriteThrough);
        }
        if constexpr (kTok == 1 && !kFp8) {
          if (hist != nullptr) {
            // first-digit histogram of the page's valid scores: each distinct
            // bin (a page's scores fall in a few dozen) is counted by the
            // lowest of its lanes, then one atomic add per bin
            const uint32_t bin = order_key(v) >> kHistShift;
            uint64_t left = __ballot(base + lane < len);
            uint32_t cnt = 0;
            while (left != 0) {
              const int l = __builtin_ctzll(left);
              const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, l);
              const uint64_t same = __ballot(bin == lb) & left;
              cnt = lane == l ? (uint32_t)__builtin_popcountll(same) : cnt;
              left &= ~same;
            }
            if (cnt != 0)
              __hip_atomic_fetch_add(hist + (int64_t)bx * kHistBins + bin, cnt, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      if constexpr (kStashed) ++stash_n;
    };

    // state at the top of each half of the loop, for the item `it` it computes:
    // its keys in KA (phase A) or KB (phase B), the id of it + 1 in flight
    Regs KA, KB;
    int bA = 0, bB = 0, bX = 0, bY = 0;
    uint32_t jA = 0, jB = 0, jX = 0, jY = 0, PX = 0, PY = 0;
    bool okA = false, okB = false, inA = false, inX = false, inY = false;
    uint32_t it = s;
    const uint32_t PA = id_load(it, bA, jA, inA);
    PY = id_load(it + 1, bY, jY, inY);
    okA = key_load(PA, inA, KA);
    for (;;) {
      // phase A: item it in KA; item it + 1's id in PY
      ensure_qw(bA);
      PX = id_load(it + 2, bX, jX, inX);
      okB = key_load(PY, inY, KB);
      bB = bY;
      jB = jY;
      compute(bA, jA, okA, KA);
      if (++it >= pe) break;
      // phase B: item it in KB; item it + 1's id in PX
      ensure_qw(bB);
      PY = id_load(it + 2, bY, jY, inY);
      okA = key_load(PX, inX, KA);
      bA = bX;
      jA = jX;
      compute(bB, jB, okB, KB);
      if (++it >= pe) break;
    }
    if constexpr (kStashed) {
      if (stash_n > 0) stash_flush();
    }
  }

  if (ts < te) {
    // -inf tail chunks
    Window W{0, 0, 0, 0, 0};
    window_set(W, first, true);
    const u32x4 ninf = {0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u};
    for (uint32_t it = ts; it < te; ++it) {
      int b;
      uint32_t c;
      window_find(W, it, sh, true, b, c);
      const RowWork r = row_work(sh, b);
      uint32_t c0 = r.tail0 + c * kTailChunk, c1 = min((uint32_t)sh.width, c0 + kTailChunk);
      if (sh.incremental) {
        // this wave owns request b's mark: the tail is [tail0, page of the old
        // mark), and the new mark is stored after the old one was read
        const uint32_t old = (uint32_t)clamp_len((int)__builtin_amdgcn_raw_buffer_load_b32(sh.marks, b * 4, 0, 0), sh.width);
        c0 = r.tail0;
        c1 = max(r.tail0, (old + kPage - 1) / kPage * kPage);
        if (lane == 0) __builtin_amdgcn_raw_buffer_store_b32(r.len, sh.marks, b * 4, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < kTok; ++t) {
        const rsrc_t row = make_rsrc(logits + ((int64_t)b * kTok + t) * sh.width, (uint32_t)sh.width * 4u);
        // c0 and c1 are multiples of 4 (page and row boundaries): whole 16-byte stores
        for (uint32_t p = c0 + 4 * lane; p < c1; p += 256)
          __builtin_amdgcn_raw_buffer_store_b128(ninf, row, p * 4, 0, kWriteThrough);
      }
    }
  }
}

// Compute units of the device `stream` runs on (queried once per device).
int cu_count(hipStream_t stream) {
  static int cached[64] = {0};
  int dev = 0;
  if (stream == nullptr || hipStreamGetDevice(stream, &dev) != hipSuccess) {
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  }
  if (dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int count = 0;
    if (hipDeviceGetAttribute(&count, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || count <= 0)
      count = 256;
    cached[dev] = count;
  }
  return cached[dev];
}

}  // namespace

namespace {

template <bool kFp8, int kTok>
void launch_variant(int grid, hipStream_t stream, const void* q, const float* w, const void* k_pool,
                    const float* k_scale, int64_t num_pages, const int32_t* page_table, const int32_t* seq_lens,
                    int32_t batch, int32_t max_pages, float* logits, int32_t* row_hwm, uint32_t* hist) {
  hipLaunchKernelGGL((score_kernel<kFp8, kTok>), dim3(grid), dim3(64), 0, stream, static_cast<const uint16_t*>(q),
                     w, k_pool, k_scale, num_pages, page_table, seq_lens, batch, max_pages, logits, row_hwm, hist);
}

}  // namespace

hipError_t launch_score(const void* q, const float* w, const void* k_pool, const float* k_scale,
                        int64_t num_pages, const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                        int32_t tokens, int32_t max_pages, float* logits, int32_t* row_hwm, uint32_t* hist,
                        hipStream_t stream) {
  // as many one-wave workgroups as stay resident, but no more than the largest
  // list these shapes allow (every slot a page, plus every tail chunk)
  const int64_t width = (int64_t)max_pages * kPage;
  const int64_t most = (int64_t)batch * max_pages + (int64_t)batch * ((width + kTailChunk - 1) / kTailChunk);
  const int per_cu = 4 * (k_scale != nullptr ? waves_per_simd<true, 1>() : waves_per_simd<false, 1>());
  const int grid = (int)std::min<int64_t>((int64_t)cu_count(stream) * per_cu, most);
  if (k_scale != nullptr) {
    launch_variant<true, 1>(grid, stream, q, w, k_pool, k_scale, num_pages, page_table, seq_lens, batch, max_pages,
                            logits, row_hwm, hist);
  } else {
    switch (tokens) {
      case 1:
        launch_variant<false, 1>(grid, stream, q, w, k_pool, k_scale, num_pages, page_table, seq_lens, batch,
                                 max_pages, logits, row_hwm, hist);
        break;
      case 2:
        launch_variant<false, 2>(grid, stream, q, w, k_pool, k_scale, num_pages, page_table, seq_lens, batch,
                                 max_pages, logits, row_hwm, nullptr);
        break;
      case 3:
        launch_variant<false, 3>(grid, stream, q, w, k_pool, k_scale, num_pages, page_table, seq_lens, batch,
                                 max_pages, logits, row_hwm, nullptr);
        break;
      default:
        launch_variant<false, 4>(grid, stream, q, w, k_pool, k_scale, num_pages, page_table, seq_lens, batch,
                                 max_pages, logits, row_hwm, nullptr);
        break;
    }
  }
  return hipGetLastError();
}

}  // namespace dsa
