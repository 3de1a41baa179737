// Sparse attention over the positions the indexer selected (page "The Indexer
// O(max_context) Breakthrough", sections "Phase 1: The MMA Sparse-MLA Decode
// Kernel" and "Phase 2: Split-K Parallelization").
//
// Every request attends with its 32 query heads over the positions of its
// top-k list. Each position holds one bfloat16 latent of 576 dims shared by
// all heads (the first 512 dims are the value). The latents sit in pages of
// 64 positions, found through the same page table as the indexer keys.
//
// attention_kernel: one 256-thread workgroup per (request, split), where a
// split is a run of at most `chunk` entries of the request's list. It
// processes tiles of 32 positions:
//   - the 32 latents are staged into LDS: each thread copies 144 B of one row
//     with 16-byte loads, and each wave's loads cover 8 rows of 128 B lines
//     per instruction. The next tile's loads are issued while the current
//     tile is being computed;
//   - S^T = K Q^T (32 positions x 32 heads) uses v_mfma_f32_32x32x16_bf16,
//     with the 576-dim contraction split over the 4 waves (9 k-steps each,
//     that wave's queries held in registers). The 4 partial tiles are summed
//     through LDS, and every wave then holds the whole S^T tile in the MFMA
//     result layout (one head per lane, 16 of the 32 positions per lane);
//   - online softmax in base 2. Per head, the running maximum is kept unless
//     a tile's maximum exceeds it by more than 8, so the output is rescaled
//     only when the maximum grows by that much (exact either way, because
//     the output and the sum of weights share the reference point);
//   - O^T += V^T P^T with the same MFMA: each wave owns 128 of the 512 value
//     dims. The weights P already sit in the B-operand layout, and V^T is
//     read from LDS with 16-bit reads.
// With one split the kernel writes the normalised output and the log-sum-exp
// directly. Otherwise it writes each split's normalised partial output and
// log-sum-exp to the workspace, and merge_kernel combines them.
//
// Workgroups are numbered so that all splits of one request, and its merge
// workgroups, run on the same XCD (workgroup i runs on XCD i % 8). A request's
// queries and partial results then stay in that XCD's L2.
#include "common.h"

namespace dsa {
namespace {

constexpr int kAttHeads = 32;
constexpr int kKD = 576;
constexpr int kVD = 512;
constexpr int kLatBytes = kKD * 2;             // one latent: 1152 B
constexpr int kLdsRow = kLatBytes + 16;        // padded LDS row: conflict-free row-wise and column-wise reads
constexpr int kTile = 32;                      // positions per tile
constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kQSteps = kKD / 16 / kAttWaves;  // 9 MFMA k-steps per wave
constexpr int kStage = kLatBytes / 128;        // 9 loads of 16 B per thread per tile
constexpr int kDimsPerWave = kVD / kAttWaves;  // 128 value dims per wave
constexpr int kMergeThreads = 256;
constexpr int kMergeParts = kAttHeads * kVD / 4 / kMergeThreads;  // 16 workgroups per request
constexpr uint32_t kSkip = 0xFFFFFFFFu;        // row code: list entry not attended
constexpr uint32_t kBad = 0xFFFFFFFEu;         // row code: entry past the table or on a page outside the pool
constexpr float kRegrow = 8.0f;                // log2 headroom before the output is rescaled
constexpr float kLn2 = 0.693147180559945309f;

static_assert(kStage * 128 == kLatBytes, "a row is 8 threads x kStage x 16 B");
static_assert(kTile * 8 == kAttThreads, "8 threads stage each row of a tile");

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

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

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// Request and split of this workgroup: workgroup i runs on XCD i % 8, so
// request b is handled by workgroups with i % 8 == b % 8.
__device__ __forceinline__ void att_place(int nsplit, int& b, int& s) {
  const int id = (int)blockIdx.x;
  const int slot = id >> 3;
  b = (slot / nsplit) * 8 + (id & 7);
  s = slot % nsplit;
}

__global__ __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attention_kernel(const AttArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kTile * kLdsRow];
  __shared__ f32x4 spart[kAttWaves * 4 * 64];
  __shared__ uint32_t rows[kMaxAttK];

  int b, s;
  att_place(a.nsplit, b, s);
  if (b >= a.batch) return;
  const int tid = (int)threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5, l32 = lane & 31;
  const int g0 = s * a.chunk;
  const int n = min(a.chunk, a.k - g0);  // list entries of this split, >= 1
  const int ntiles = (n + kTile - 1) / kTile;

  // Resolve every entry of the split to a pool row (page * 64 + slot row).
  const rsrc_t ir = make_rsrc(a.idx + (int64_t)b * a.k, (uint32_t)a.k * 4u);
  const rsrc_t pr = make_rsrc(a.page_table + (int64_t)b * a.max_pages, (uint32_t)a.max_pages * 4u);
  const int width = a.max_pages * kPage;
  int bad = 0;
  for (int u = tid; u < ntiles * kTile; u += kAttThreads) {
    uint32_t v = kSkip;
    if (u < n) {
      const int pos = (int)load_u32(ir, (g0 + u) * 4);
      if (pos >= width) {
        v = kBad;
      } else if (pos >= 0) {
        const int page = (int)load_u32(pr, (pos >> 6) * 4);
        v = (page < 0 || (int64_t)page >= a.num_pages) ? kBad : (uint32_t)page * kPage + (uint32_t)(pos & 63);
      }
    }
    bad |= v == kBad;
    rows[u] = v;
  }

  // This wave's slice of the queries: B operand of k-steps 9*wv .. 9*wv+8.
  const rsrc_t qr = make_rsrc(a.q + (int64_t)b * kAttHeads * kKD, kAttHeads * kLatBytes);
  u32x4 qv[kQSteps];
#pragma unroll
  for (int j = 0; j < kQSteps; ++j)
    qv[j] = __builtin_amdgcn_raw_buffer_load_b128(qr, l32 * kLatBytes + (2 * (kQSteps * wv + j) + hf) * 16, 0, 0);

  bad = __syncthreads_or(bad);  // also publishes rows[]

  // Staging: thread tid copies bytes [16*(tid%8) + 128*i, +16) of tile row tid/8.
  const int srow = tid >> 3, scol = (tid & 7) * 16;
  u32x4 R[kStage];
  auto stage_load = [&](int t) {
    const uint32_t v = rows[t * kTile + srow];
    const uint64_t row = v >= kBad ? 0u : v;  // skipped and bad entries read row 0 (never used)
    const unsigned char* src = reinterpret_cast<const unsigned char*>(a.kv) + row * kLatBytes + scol;
#pragma unroll
    for (int i = 0; i < kStage; ++i)
      R[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 128 * i));
  };
  stage_load(0);

  f32x16 O[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[t4][r] = 0.f;
  float m_run = -__builtin_inff(), l_run = 0.f;

  const unsigned char* kbase = tile + l32 * kLdsRow + hf * 16 + kQSteps * wv * 32;
  const unsigned char* vbase = tile + 4 * hf * kLdsRow + 2 * l32 + 2 * kDimsPerWave * wv;
  unsigned char* sdst = tile + srow * kLdsRow + scol;

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done with the previous tile's LDS
#pragma unroll
    for (int i = 0; i < kStage; ++i) *reinterpret_cast<u32x4*>(sdst + 128 * i) = R[i];
    __syncthreads();
    if (t + 1 < ntiles) stage_load(t + 1);

    // Partial S^T over this wave's 144 dims.
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
    for (int j = 0; j < kQSteps; ++j) S = mfma(*reinterpret_cast<const u32x4*>(kbase + 32 * j), qv[j], S);
#pragma unroll
    for (int g = 0; g < 4; ++g) spart[(wv * 4 + g) * 64 + lane] = f32x4{S[4 * g], S[4 * g + 1], S[4 * g + 2], S[4 * g + 3]};
    const uint32_t mask = (uint32_t)__ballot(rows[t * kTile + l32] < kBad);
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v = spart[g * 64 + lane];
#pragma unroll
      for (int w2 = 1; w2 < kAttWaves; ++w2) v += spart[(w2 * 4 + g) * 64 + lane];
      S[4 * g] = v[0], S[4 * g + 1] = v[1], S[4 * g + 2] = v[2], S[4 * g + 3] = v[3];
    }

    // Lane (head l32, half hf) register r holds tile position 8(r/4) + 4hf + r%4.
    const uint32_t ml = mask >> (4 * hf);
    float mt = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[r] = ((ml >> (8 * (r >> 2) + (r & 3))) & 1u) ? S[r] * a.c : -__builtin_inff();
      mt = fmaxf(mt, S[r]);
    }
    mt = fmaxf(mt, xor32(mt));
    if (__any(mt > m_run + kRegrow)) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) O[t4] *= alpha;
      l_run *= alpha;
      m_run = mn;
    }
    const float ref = m_run == -__builtin_inff() ? 0.f : m_run;
    u32x4 P[2];
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const __bf16 p0 = (__bf16)__builtin_amdgcn_exp2f(S[r] - ref);
      const __bf16 p1 = (__bf16)__builtin_amdgcn_exp2f(S[r + 1] - ref);
      lsum += (float)p0 + (float)p1;
      P[r >> 3][(r >> 1) & 3] = (uint32_t)__builtin_bit_cast(uint16_t, p0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, p1) << 16);
    }
    l_run += lsum;

    // O^T[dims of this wave] += V^T P^T; k-slot (hf, i) of step js is tile
    // position 16js + 8(i/4) + 4hf + i%4, matching P's layout.
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        u16x8 e;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          e[i] = *reinterpret_cast<const uint16_t*>(vbase + (16 * js + 8 * (i >> 2) + (i & 3)) * kLdsRow + 64 * t4);
        O[t4] = mfma(__builtin_bit_cast(u32x4, e), P[js], O[t4]);
      }
    }
  }

  // Finish: sum of weights over both halves, normalise, log-sum-exp (natural log).
  const float l_tot = l_run + xor32(l_run);
  float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  float lse_v = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -__builtin_inff();
  if (bad) inv = lse_v = __builtin_nanf("");
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
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = f32x4{O[t4][4 * g], O[t4][4 * g + 1], O[t4][4 * g + 2], O[t4][4 * g + 3]} * inv;
      const int d = kDimsPerWave * wv + 32 * t4 + 8 * g + 4 * hf;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), orr, (l32 * kVD + d) * 4, 0, 0);
    }
  if (wv == 0 && hf == 0) {
    const rsrc_t lr = make_rsrc(dst_l, kAttHeads * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, lse_v), lr, l32 * 4, 0, 0);
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
  float M = -__builtin_inff();
  bool nan = false;
  for (int s = 0; s < ns; ++s) {
    const float x = __builtin_bit_cast(float, load_u32(lr, (s * kAttHeads + h) * 4));
    nan |= x != x;
    M = fmaxf(M, x);
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (M > -__builtin_inff()) {
    for (int s = 0; s < ns; ++s) {
      const float x = __builtin_bit_cast(float, load_u32(lr, (s * kAttHeads + h) * 4));
      const float wt = __builtin_amdgcn_exp2f((x - M) * 1.44269504088896341f);
      const f32x4 o = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(orr, ((s * kAttHeads + h) * kVD + d) * 4, 0, 0));
      acc += o * wt;
      wsum += wt;
    }
  }
  float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  float l = wsum > 0.f ? M + __builtin_amdgcn_logf(wsum) * kLn2 : -__builtin_inff();
  if (nan) inv = l = __builtin_nanf("");
  const rsrc_t out = make_rsrc(a.out + ((int64_t)b * kAttHeads + h) * kVD, kVD * 4);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc * inv), out, d * 4, 0, 0);
  if (d == 0) {
    const rsrc_t lo = make_rsrc(a.lse + (int64_t)b * kAttHeads, kAttHeads * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), lo, h * 4, 0, 0);
  }
}

}  // namespace

void att_plan(int32_t batch, int32_t k, int32_t* nsplit, int32_t* chunk) {
  const int tiles = (k + kTile - 1) / kTile;
  const int want = max(1, min(tiles, (kAttTargetGroups + batch - 1) / batch));
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
