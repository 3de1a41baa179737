// Sparse attention over the positions the indexer selected (page "The Indexer
// O(max_context) Breakthrough", sections "Phase 1: The MMA Sparse-MLA Decode
// Kernel" and "Phase 2: Split-K Parallelization").
//
// Every request attends with its 32 query heads over the positions of its
// top-k list. Each position holds one bfloat16 latent of 576 dims shared by
// all heads (the first 512 dims are the value). The latents sit in pages of
// 64 positions, found through the same page table as the indexer keys.
//
// attention_kernel: one 512-thread workgroup per (request, split), where a
// split is a run of at most `chunk` entries of the request's list, on one CU:
// four compute waves and four loader waves, two waves per SIMD. It processes
// tiles of 32 positions:
//   - staging (the loader waves): direct-to-LDS loads (global_load_lds_dwordx4)
//     into four tile buffers, up to four tiles ahead. Rows are stored as 72
//     chunks of 16 B, with chunk c of row r at c ^ swz(r);
//   - scores: wave (ph, hh) computes the 16 positions x 16 heads block
//     (positions 16ph.., heads 16hh..) of S^T over the 576 dims with
//     v_mfma_f32_16x16x32_bf16 (its 16 heads' queries held in registers) and
//     publishes it with its per-head maxima to a score tile in LDS;
//   - softmax: every wave reads the whole 32 x 32 score tile and runs the same
//     online softmax in base 2, so no other agreement between waves is
//     needed; the output is rescaled only when a head's maximum grows by more
//     than 8 (exact either way, as the output and the sum of weights share
//     the reference). The weights, rounded to bf16, sit in the registers in
//     the B-operand layout of the value product;
//   - values: wave wv owns value dims 128wv..128wv+127 for all 32 heads:
//     O^T (16 dims x 16 heads blocks) += V^T P^T on 16x16x32 MFMAs, V^T read
//     straight from the staged rows with ds_read_b64_tr_b16 (each 16-lane
//     group reads a 4 x 16 block of bf16 and receives it transposed); each
//     transposed read feeds both head blocks.
// The steps are software-pipelined (the softmax of tile t, the scores of tile
// t+1 and the values of tile t in one step), with one barrier per tile.
// With one split the kernel writes the normalised output and the log-sum-exp
// directly. Otherwise it writes each split's normalised partial output and
// log-sum-exp to the workspace, and merge_kernel combines them.
//
// Workgroups are numbered so that all splits of one request, and its merge
// workgroups, run on the same XCD (workgroup i runs on XCD i % 8). A request's
// queries and partial results then stay in that XCD's L2. Both kernels store
// their results written through the L2 (kWriteThrough), so that the end of a
// kernel has no dirty lines to write back before the next one starts
// (measured against ordinary stores: a call at B = 64, k = 2048 is 1.1-1.8 us
// faster).
#include "common.h"

namespace dsa {
namespace {

constexpr int kAttHeads = 32;
constexpr int kKD = 576;
constexpr int kVD = 512;
constexpr int kLatBytes = kKD * 2;             // one latent: 1152 B = 72 chunks of 16 B
constexpr int kTile = 32;                      // positions per tile
constexpr int kTileBytes = kTile * kLatBytes;  // 36 KiB
constexpr int kBufs = 4;                       // staged tiles: one computed, three loading
constexpr int kSRow = 36;                      // floats per row (head) of the score tile: 32 + padding
constexpr int kSTile = kAttHeads * kSRow;
constexpr int kWorkThreads = 256;             // the four compute waves
constexpr int kAttThreads = 2 * kWorkThreads;  // and four loader waves
constexpr int kQSteps = kKD / 32;              // 18 k-steps of the 16x16x32 MFMA
constexpr int kStage = kLatBytes / 128;        // 9 loads of 16 B per thread per tile
constexpr int kMergeThreads = 256;
constexpr int kMergeParts = kAttHeads * kVD / 4 / kMergeThreads;  // 16 workgroups per request
constexpr int kMergeBatch = 8;                 // splits whose partials one merge thread loads at once
constexpr uint32_t kSkip = 0xFFFFFFFFu;        // row code: list entry not attended
constexpr uint32_t kBad = 0xFFFFFFFEu;         // row code: entry past the table or on a page outside the pool
constexpr float kRegrow = 8.0f;                // log2 headroom of the weights over the running maximum
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kStage * 128 == kLatBytes, "a row is 8 threads x kStage x 16 B");
static_assert(kTile * 8 == kWorkThreads, "8 loader lanes stage each row of a tile");
static_assert(kMaxAttChunk % kTile == 0, "splits are whole tiles");

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

struct AttArgs {
  const uint16_t* q;          // [batch][32][576] bf16
  const uint16_t* kv;         // [num_pages][64][576] bf16
  int64_t num_pages;
  const int32_t* page_table;  // [batch][max_pages]
  const int32_t* idx;         // [batch][k]
  float* out;                 // [batch][32][512]
  float* lse;                 // [batch][32]
  float* part_o;              // [batch][nsplit][32][512] (nsplit > 1)
  float* part_lse;            // [batch][nsplit][32]
  float c;                    // softmax scale * log2(e)
  int32_t max_pages, k, batch, nsplit, chunk;
};

__device__ __forceinline__ uint32_t load_u32(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Combine v over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with op, in
// registers: v_permlane32_swap of two copies of v leaves lane l's value and
// lane l ^ 32's in the pair; v_permlane16_swap then does the same across
// rows of 16 lanes.
template <typename Op>
__device__ __forceinline__ float xor_lanes_16_32(float v, Op op) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float w = op(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t x = __builtin_bit_cast(uint32_t, w);
  const auto b = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

// Chunk c of staged row r sits at chunk c ^ (r & 7) of that row: the rows of
// an aligned group of 8 put any given chunk in 8 different 16-byte slots of
// one 128-byte span. Measured on gfx950 with the kernel's access patterns:
// the 16-row score reads then run at the speed of contiguous 16-byte reads,
// and the transposed value reads at their own full rate.
__device__ __forceinline__ int swz(int r) { return r & 7; }

// 4 bf16 of LDS, transposed across each 16-lane group.
__device__ __forceinline__ u32x2 read_tr(const unsigned char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b, float& sum) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;
  sum += (float)x + (float)y;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Request and split of this workgroup: workgroup i runs on XCD i % 8, so
// request b is handled by workgroups with i % 8 == b % 8.
__device__ __forceinline__ void att_place(int nsplit, int& b, int& s) {
  const int id = (int)blockIdx.x;
  const int slot = id >> 3;
  b = (slot / nsplit) * 8 + (id & 7);
  s = slot % nsplit;
}

// Direct-to-LDS load of 16 B per lane: lane l's bytes land at lds + 16 l
// (lds is a wave-uniform LDS byte address). Issued as inline assembly so that the compiler does
// not track it: its completion is awaited explicitly (s_waitcnt vmcnt, then a
// barrier) before any wave reads the buffer. Extra outstanding loads can only
// make the compiler's own vmcnt waits stricter, never looser. m0 is listed as
// clobbered, so the compiler keeps no value of its own there across the load
// (it reserves m0 and warns that a reserved register is named; the warning is
// silenced here only).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Encoding of s_waitcnt that waits until at most n vector-memory operations
// and no LDS operations of this wave are outstanding.
constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8); }

__global__ __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(const AttArgs a) {
  // Tile t is staged in buffer t % 4 while tiles t+1 .. t+3 are loading.
  __shared__ __attribute__((aligned(16))) unsigned char tbuf[kBufs * kTileBytes];
  __shared__ __attribute__((aligned(16))) float sbuf[2 * kSTile];  // score tiles of two consecutive tiles
  __shared__ float mbuf[2][2][kAttHeads];                           // [tile % 2][position half][head] maxima
  __shared__ uint32_t rows[kMaxAttChunk];

  int b, s;
  att_place(a.nsplit, b, s);
  if (b >= a.batch) return;
  const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool loader = wv >= kWorkThreads / 64;  // waves 4..7 only stage tiles
  const int g0 = s * a.chunk;
  const int n = min(a.chunk, a.k - g0);  // list entries of this split, >= 1
  const int ntiles = (n + kTile - 1) / kTile;

  // Wave (hh, dh): heads 16hh..16hh+15, value dims 256dh..256dh+255.
  // Lane (g, j): column/row j of every 16x16 block, k-slots 8g..8g+7.
  const int g = lane >> 4, j = lane & 15;
  const rsrc_t qr = make_rsrc(a.q + (int64_t)b * kAttHeads * kKD, kAttHeads * kLatBytes);
  u32x4 qv[kQSteps];  // queries of head 16(wv >> 1) + j, k-slots 8g.. of each 32-dim step
  if (!loader) {
#pragma unroll
    for (int st = 0; st < kQSteps; ++st)
      qv[st] = __builtin_amdgcn_raw_buffer_load_b128(qr, (16 * (wv >> 1) + j) * kLatBytes + (4 * st + g) * 16, 0, 0);
  }

  // Resolve every entry of the split to a pool row (page * 64 + slot row).
  const rsrc_t ir = make_rsrc(a.idx + (int64_t)b * a.k, (uint32_t)a.k * 4u);
  const rsrc_t pr = make_rsrc(a.page_table + (int64_t)b * a.max_pages, (uint32_t)a.max_pages * 4u);
  // Every entry load of the lane first, then every page-table load: two
  // memory round trips in all, whatever the number of entries per lane.
  const int width = a.max_pages * kPage;
  constexpr int kPer = kMaxAttChunk / kAttThreads;  // entries per lane, at most
  static_assert(kPer * kAttThreads == kMaxAttChunk, "entries per lane");
  int pos[kPer], page[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid + i * kAttThreads;
    pos[i] = u < n ? (int)load_u32(ir, (g0 + u) * 4) : -1;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool need = pos[i] >= 0 && pos[i] < width;
    page[i] = need ? (int)load_u32(pr, (pos[i] >> 6) * 4) : 0;
  }
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int u = tid + i * kAttThreads;
    if (u < ntiles * kTile) {
      uint32_t v = kSkip;
      if (pos[i] >= width) {
        v = kBad;
      } else if (pos[i] >= 0) {
        v = (page[i] < 0 || (int64_t)page[i] >= a.num_pages) ? kBad
                                                            : (uint32_t)page[i] * kPage + (uint32_t)(pos[i] & 63);
      }
      bad |= v == kBad;
      rows[u] = v;
    }
  }
  bad = __syncthreads_or(bad);  // also publishes rows[]

  // Staging with direct-to-LDS loads: loader wave lw's load i fills LDS
  // chunks 64(9lw + i) .. +63 of the tile (lane -> +lane). LDS chunk L is row
  // L / 72, stored position L % 72, which holds row chunk (L % 72) ^ swz(row).
  const int lw = wv & 3;
  int drow[kStage], dsrc[kStage];
#pragma unroll
  for (int i = 0; i < kStage; ++i) {
    const int L = 64 * (kStage * lw + i) + lane;
    const int r = L / 72, p = L % 72;
    drow[i] = r;
    dsrc[i] = ((p & ~7) | ((p & 7) ^ swz(r))) * 16;
  }
  const unsigned char* kvb = reinterpret_cast<const unsigned char*>(a.kv);
  const uint32_t lds_tiles =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)tbuf + 1024u * kStage * lw;
  auto stage = [&](int buf, int t) {
    uint32_t v[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) v[i] = rows[t * kTile + drow[i]];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const uint64_t row = v[i] >= kBad ? 0u : v[i];  // skipped and bad entries read row 0 (never used)
      dma16(kvb + row * kLatBytes + dsrc[i],
            __builtin_amdgcn_readfirstlane(lds_tiles + (uint32_t)(buf * kTileBytes + 1024 * i)));
    }
  };

  // Scores: wave (ph, hh) computes S^T for tile positions 16ph..16ph+15 and
  // heads 16hh..16hh+15 over the 576 dims (v_mfma_f32_16x16x32_bf16, lane
  // (g, j): row/column j, k-slots 8g..8g+7). It publishes the block and its
  // per-head maximum; after a barrier every wave reads back the whole 32 x 32
  // tile and runs the same softmax, so no other agreement is needed.
  const int ph = wv & 1, hh = wv >> 1;
  const int kofs_even = (16 * ph + j) * kLatBytes + ((g ^ swz(j)) * 16);
  const int kofs_odd = (16 * ph + j) * kLatBytes + (((4 + g) ^ swz(j)) * 16);
  const int s_wr = (16 * hh + j) * kSRow + 16 * ph + 4 * g;  // floats into sbuf

  // Values: wave wv owns dims 128wv..128wv+127 for all 32 heads: O^T blocks
  // (16 dims x 16 heads) for dim block db and head block hb. A = V^T via
  // ds_read_b64_tr_b16: lane (g, kk, aa) reads tile row 8g + 4ld + kk at dims
  // d0 + 4aa .. +3 of block d0 = 128wv + 16db; B = P^T: k-slot (g, i) is tile
  // position 8g + i.
  const int kk = (lane & 15) >> 2, aa = lane & 3;
  int vb[2];  // [ld]: tile row 8g + 4ld + kk, dims of block 0 (swizzle applied per block below)
  int vx[2][4];
#pragma unroll
  for (int ld = 0; ld < 2; ++ld) {
    const int r = 8 * g + 4 * ld + kk;
    vb[ld] = r * kLatBytes + 16 * (16 * wv) + 8 * (aa & 1);
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) vx[ld][m4] = ((2 * m4 + (aa >> 1)) ^ swz(r)) * 16;
  }

  f32x4 O[2][8];  // [hb][db]: dims 128wv + 16db + 4g + r, head 16hb + j
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int db = 0; db < 8; ++db) O[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-__builtin_inff(), -__builtin_inff()}, l_run[2] = {0.f, 0.f};

  // Scores of tile t (this wave's 16 x 16 block) into score buffer t % 2.
  auto scores = [&](const unsigned char* cur, int t) {
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = S0;
#pragma unroll
    for (int s0 = 0; s0 < kQSteps; s0 += 6) {  // six operand reads in flight, then six MFMAs
      u32x4 kx[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int st = s0 + i;
        kx[i] = *reinterpret_cast<const u32x4*>(cur + ((st & 1) ? kofs_odd : kofs_even) + 64 * (st & ~1));
      }
#pragma unroll
      for (int i = 0; i < 6; i += 2) {
        S0 = mfma16(kx[i], qv[s0 + i], S0);
        S1 = mfma16(kx[i + 1], qv[s0 + i + 1], S1);
      }
    }
    // Register r: tile position 16ph + 4g + r, head 16hh + j.
    const uint32_t mask = (uint32_t)__ballot(rows[t * kTile + (lane & 31)] < kBad);
    f32x4 S = S0 + S1;
    const uint32_t mine = mask >> (16 * ph + 4 * g);
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      S[r] = ((mine >> r) & 1u) ? S[r] * a.c : -__builtin_inff();
      mt = fmaxf(mt, S[r]);
    }
    mt = xor_lanes_16_32(mt, [](float x, float y) { return fmaxf(x, y); });
    *reinterpret_cast<f32x4*>(sbuf + (t & 1) * kSTile + s_wr) = S;
    if (g == 0) mbuf[t & 1][ph][16 * hh + j] = mt;
  };

  // Softmax of tile t (score buffer t % 2, complete in every wave) for heads
  // j (hb = 0) and 16 + j (hb = 1) at this lane's positions 8g..8g+7: the
  // B operands of the value product, rescaling O when a maximum grows.
  auto softmax = [&](int t, u32x4 (&P)[2]) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int h = 16 * hb + j;
      const float* sb = sbuf + (t & 1) * kSTile + h * kSRow + 8 * g;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(sb);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(sb + 4);
      const float tm = fmaxf(mbuf[t & 1][0][h], mbuf[t & 1][1][h]);
      if (__any(tm > m_run[hb] + kRegrow)) {
        const float mn = fmaxf(m_run[hb], tm);
        const float alpha = m_run[hb] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run[hb] - mn);
#pragma unroll
        for (int db = 0; db < 8; ++db) O[hb][db] *= alpha;
        l_run[hb] *= alpha;
        m_run[hb] = mn;
      }
      const float ref = m_run[hb] == -__builtin_inff() ? 0.f : m_run[hb];
      P[hb][0] = pack_bf16(__builtin_amdgcn_exp2f(x0[0] - ref), __builtin_amdgcn_exp2f(x0[1] - ref), l_run[hb]);
      P[hb][1] = pack_bf16(__builtin_amdgcn_exp2f(x0[2] - ref), __builtin_amdgcn_exp2f(x0[3] - ref), l_run[hb]);
      P[hb][2] = pack_bf16(__builtin_amdgcn_exp2f(x1[0] - ref), __builtin_amdgcn_exp2f(x1[1] - ref), l_run[hb]);
      P[hb][3] = pack_bf16(__builtin_amdgcn_exp2f(x1[2] - ref), __builtin_amdgcn_exp2f(x1[3] - ref), l_run[hb]);
    }
  };

  // O^T += V^T P^T over tile `cur`: each V^T block feeds both head blocks.
  auto values = [&](const unsigned char* cur, const u32x4 (&P)[2]) {
#pragma unroll
    for (int d0 = 0; d0 < 8; d0 += 4) {
      u32x4 va[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int db = d0 + i;
        const u32x2 lo = read_tr(cur + vb[0] + 128 * (db >> 2) + vx[0][db & 3]);
        const u32x2 hi = read_tr(cur + vb[1] + 128 * (db >> 2) + vx[1][db & 3]);
        va[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        O[0][d0 + i] = mfma16(va[i], P[0], O[0][d0 + i]);
        O[1][d0 + i] = mfma16(va[i], P[1], O[1][d0 + i]);
      }
    }
  };

  // Software pipeline over the tiles, one barrier per step, in which the
  // loader waves and the compute waves meet. Compute step t: the softmax of
  // tile t (its scores were published in step t-1), the scores of tile t+1
  // and the values of tile t, three independent streams the compiler
  // interleaves; then its LDS accesses are waited for and the barrier
  // follows. Loader step t: wait for its loads of tile t+2, the barrier (tile
  // t+1's scores are complete, tile t+2 has landed, every wave is done with
  // tile t), then refill tile t's buffer with tile t+4. The prologue loads
  // tiles 0..3 and publishes tile 0's scores. (Issuing the loads from the
  // compute waves stalled them on the memory pipeline's back-pressure, about
  // 950 cycles per tile.) Both roles pass the same 2 + ntiles barriers.
  auto tbuf_of = [&](int t) { return tbuf + (t & (kBufs - 1)) * kTileBytes; };
  const int later = min(kBufs, ntiles) - 1;  // tiles 1.. loading in the prologue
  if (loader) {
    for (int t = 0; t < kBufs && t < ntiles; ++t) stage(t, t);
    // tile 0 has landed
    if (later >= 3)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(3 * kStage));
    else if (later == 2)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * kStage));
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kStage));
    else
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    __builtin_amdgcn_s_barrier();
    // tile 1 has landed
    if (later >= 3)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(2 * kStage));
    else if (later == 2)
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kStage));
    else
      __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    __builtin_amdgcn_s_barrier();
    for (int t = 0; t < ntiles; ++t) {
      // tile t+2 must have landed; tile t+3's loads may still be in flight
      if (t + 3 < ntiles)
        __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(kStage));
      else
        __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
      __builtin_amdgcn_s_barrier();
      if (t + kBufs < ntiles) stage(t & (kBufs - 1), t + kBufs);
    }
    return;
  }
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));  // the queries have landed
  __builtin_amdgcn_s_barrier();
  scores(tbuf_of(0), 0);
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
  __builtin_amdgcn_s_barrier();
  for (int t = 0; t < ntiles; ++t) {
    u32x4 P[2];
    softmax(t, P);
    if (t + 1 < ntiles) scores(tbuf_of(t + 1), t + 1);
    values(tbuf_of(t), P);
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
    __builtin_amdgcn_s_barrier();
  }

  // Sums of weights of this lane's two heads over all lanes (g) of the wave.
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    l_run[hb] = xor_lanes_16_32(l_run[hb], [](float x, float y) { return x + y; });
  }
  float* dst_o;
  float* dst_l;
  if (a.nsplit == 1) {
    dst_o = a.out + (int64_t)b * kAttHeads * kVD;
    dst_l = a.lse + (int64_t)b * kAttHeads;
  } else {
    const int64_t part = (int64_t)b * a.nsplit + s;
    dst_o = a.part_o + part * kAttHeads * kVD;
    dst_l = a.part_lse + part * kAttHeads;
  }
  const rsrc_t orr = make_rsrc(dst_o, kAttHeads * kVD * 4);
  const rsrc_t lr = make_rsrc(dst_l, kAttHeads * 4);
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = 16 * hb + j;
    const float inv = bad ? __builtin_nanf("") : (l_run[hb] > 0.f ? 1.0f / l_run[hb] : 0.f);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 128 * wv + 16 * db + 4 * g;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, O[hb][db] * inv), orr, (h * kVD + d) * 4, 0, kWriteThrough);
    }
    if (wv == 0 && g == 0) {
      float lse_v = l_run[hb] > 0.f ? (m_run[hb] + __builtin_amdgcn_logf(l_run[hb])) * kLn2 : -__builtin_inff();
      if (bad) lse_v = __builtin_nanf("");
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), lr, h * 4, 0, kWriteThrough);
    }
  }
}

// Combines the splits of each (request, head): with M the largest split
// log-sum-exp, weight_s = exp(lse_s - M); out = sum_s weight_s * o_s / sum_s
// weight_s and lse = M + log(sum_s weight_s). 16 workgroups per request, each
// covering 2 heads x 512 dims with one float4 per thread.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const AttArgs a) {
  const int id = (int)blockIdx.x;
  const int slot = id >> 3;
  const int b = (slot / kMergeParts) * 8 + (id & 7);
  if (b >= a.batch) return;
  const int part = slot % kMergeParts;
  const int tid = (int)threadIdx.x;
  const int h = part * (kMergeThreads * 4 / kVD) + tid / (kVD / 4);
  const int d = (tid % (kVD / 4)) * 4;
  const int ns = a.nsplit;
  const rsrc_t lr = make_rsrc(a.part_lse + (int64_t)b * ns * kAttHeads, (uint32_t)ns * kAttHeads * 4u);
  const rsrc_t orr = make_rsrc(a.part_o + (int64_t)b * ns * kAttHeads * kVD, (uint32_t)ns * kAttHeads * kVD * 4u);
  // The partial outputs are loaded with the log-sum-exps (eight splits at a
  // time), not after their maximum is known: one memory round trip, not two.
  float M = -__builtin_inff();
  bool nan = false;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float x[kMergeBatch];
    f32x4 o[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int sx = min(s0 + i, ns - 1);  // repeats of the last split are not accumulated
      x[i] = __builtin_bit_cast(float, load_u32(lr, (sx * kAttHeads + h) * 4));
      o[i] = __builtin_bit_cast(f32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(orr, ((sx * kAttHeads + h) * kVD + d) * 4, 0, 0));
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      if (s0 + i < ns) {
        nan |= x[i] != x[i];
        Mb = fmaxf(Mb, x[i]);
      }
    }
    if (Mb > -__builtin_inff()) {
      // rebase what was accumulated so far to the new maximum, then add this batch
      const float r = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((M - Mb) * 1.44269504088896341f);
      acc *= r;
      wsum *= r;
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        if (s0 + i < ns) {
          const float wt = __builtin_amdgcn_exp2f((x[i] - Mb) * 1.44269504088896341f);
          acc += o[i] * wt;
          wsum += wt;
        }
      }
    }
    M = Mb;
  }
  float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  float l = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -__builtin_inff();
  if (nan) inv = l = __builtin_nanf("");
  const rsrc_t out = make_rsrc(a.out + ((int64_t)b * kAttHeads + h) * kVD, kVD * 4);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc * inv), out, d * 4, 0, kWriteThrough);
  if (d == 0) {
    const rsrc_t lo = make_rsrc(a.lse + (int64_t)b * kAttHeads, kAttHeads * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), lo, h * 4, 0, kWriteThrough);
  }
}

}  // namespace

void att_plan(int32_t batch, int32_t k, int32_t* nsplit, int32_t* chunk) {
  const int tiles = (k + kTile - 1) / kTile;
  const int want = max((tiles * kTile + kMaxAttChunk - 1) / kMaxAttChunk,
                       max(1, min(tiles, (kAttTargetGroups + batch - 1) / batch)));
  const int per = (tiles + want - 1) / want;
  *chunk = per * kTile;
  *nsplit = (tiles + per - 1) / per;
}

size_t att_workspace_bytes(int32_t batch, int32_t k) {
  int32_t nsplit, chunk;
  att_plan(batch, k, &nsplit, &chunk);
  if (nsplit == 1) return 0;
  return (size_t)batch * nsplit * kAttHeads * (kVD + 1) * sizeof(float);
}

hipError_t launch_attention(const void* q, const void* kv, int64_t num_pages, const int32_t* page_table,
                            int32_t batch, int32_t max_pages, const int32_t* idx, int32_t k, float scale,
                            float* out, float* lse, void* workspace, hipStream_t stream) {
  AttArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.num_pages = num_pages;
  a.page_table = page_table;
  a.idx = idx;
  a.out = out;
  a.lse = lse;
  a.c = scale * 1.44269504088896341f;
  a.max_pages = max_pages;
  a.k = k;
  a.batch = batch;
  att_plan(batch, k, &a.nsplit, &a.chunk);
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = a.nsplit > 1 ? a.part_o + (size_t)batch * a.nsplit * kAttHeads * kVD : nullptr;
  const int groups8 = (batch + 7) / 8;
  hipLaunchKernelGGL(attention_kernel, dim3(groups8 * 8 * a.nsplit), dim3(kAttThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(groups8 * 8 * kMergeParts), dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
