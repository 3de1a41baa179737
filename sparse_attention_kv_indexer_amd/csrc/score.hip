// Score kernel of the DSA indexer decode step on gfx950.
//
// What it computes (page "The O(Actual) Indexer", section "The Bottleneck That
// Was"; page "The Moment of Breakthrough", section "The Context"): for request
// b and every c4 position s below its length,
//     logits[b][s] = sum_h w[b][h] * max(0, q[b][h] . k[page_table[b][s/64]][s%64])
// and -inf at every position at or past the length, over a row of
// max_pages * 64 positions.
//
// Launch shape: one 64-lane workgroup per (page slot, request), a grid fixed by
// (max_pages, batch) so the launch can be captured once and replayed for any
// lengths. A workgroup whose slot lies wholly past the length takes the early
// exit of the section "The Benchmark Results": it reads neither the page table
// nor the key page and only writes 64 x -inf (or nothing, in the incremental
// mode, when the page is already -inf). Work and HBM traffic therefore follow
// the actual length; only the 4-byte output per position follows the row width.
//
// A valid slot reads its 8 KiB key page with eight fully coalesced 1 KiB wave
// loads, stages it in LDS under an XOR swizzle, and contracts it against the
// request's 32 x 64 query block with eight v_mfma_f32_32x32x16_bf16 (bf16
// products, fp32 accumulation). The accumulator holds the 32 heads x 32
// positions of each half page with one position per lane; ReLU, the head
// weights and 16 of the 32 heads are summed in registers, and one cross-half
// lane exchange adds the other 16 heads.
#include "common.h"

namespace dsa {
namespace {

__device__ __forceinline__ int clamp_len(int len, int width) { return min(max(len, 0), width); }

// LDS slot of 16-byte chunk `col` (0..7) of key row `row` (0..63). Each key row
// is 128 B; XOR-ing the chunk index with the row keeps the eight rows read by
// consecutive lanes of an MFMA operand load on distinct banks.
__device__ __forceinline__ int lds_slot(int row, int col) { return row * 8 + (col ^ (row & 7)); }

__global__ __launch_bounds__(64) void score_kernel(
    const uint16_t* __restrict__ q,          // bf16 [B][32][64]
    const float* __restrict__ w,             // [B][32]
    const uint16_t* __restrict__ k_pool,     // bf16 [num_pages][64][64]
    int64_t num_pages,
    const int32_t* __restrict__ page_table,  // [B][max_pages]
    const int32_t* __restrict__ seq_lens,    // [B]
    int32_t max_pages,
    float* __restrict__ logits,              // [B][max_pages * 64]
    const int32_t* __restrict__ row_hwm)     // [B] or null
{
  const int slot = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int width = max_pages * kPage;
  const int len = clamp_len(seq_lens[b], width);
  const int base = slot * kPage;
  const rsrc_t out = make_rsrc(logits + (int64_t)b * width + base, kPage * sizeof(float));

  float val = -__builtin_inff();
  if (base >= len) {
    // early exit: the whole page is past the length; no page-table or key read
    if (row_hwm != nullptr && base >= clamp_len(row_hwm[b], width)) return;  // already -inf
  } else {
    const int page = page_table[(int64_t)b * max_pages + slot];
    if (page < 0 || (int64_t)page >= num_pages) {
      // a page id outside the pool is never dereferenced
      val = __builtin_nanf("");
    } else {
      // key page: 16-byte chunk c = 64 * i + lane is key row c / 8, column c % 8;
      // each i is one fully coalesced 1 KiB wave load
      const rsrc_t kp = make_rsrc(k_pool + (int64_t)page * (kPage * kDim), kPageBytes);
      u32x4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(kp, (i * 64 + lane) * 16, 0, kNonTemporal);

      // query operand A (32 heads x 16 dims per step): lane holds head lane%32,
      // dims 16*kb + 8*(lane/32) .. +7 = chunk 2*kb + lane/32 of that head's row
      const int half = lane >> 5;
      const int n = lane & 31;
      const rsrc_t qr = make_rsrc(q + (int64_t)b * (kHeads * kDim), kHeads * kRowBytes);
      bf16x8 a[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        a[kb] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, n * kRowBytes + (2 * kb + half) * 16, 0, 0));

      // head weights in accumulator order: register r of a lane holds head
      // 8*(r/4) + 4*half + r%4, so group g = r/4 is the float4 at head 8*g + 4*half
      const rsrc_t wr = make_rsrc(w + (int64_t)b * kHeads, kHeads * sizeof(float));
      f32x4 wv[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        wv[g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, (8 * g + 4 * half) * 4, 0, 0));

      __shared__ u32x4 tile[kPageChunks];
#pragma unroll
      for (int i = 0; i < 8; ++i) tile[lds_slot(i * 8 + (lane >> 3), lane & 7)] = v[i];
      __syncthreads();

      // keys operand B (16 dims x 32 positions per step): lane holds position
      // lane%32 of the half page, dims 16*kb + 8*half .. +7
      f32x16 acc0 = {};  // positions 0..31 of the page
      f32x16 acc1 = {};  // positions 32..63
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int col = 2 * kb + half;
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, tile[lds_slot(n, col)]);
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, tile[lds_slot(n + 32, col)]);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], b0, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kb], b1, acc1, 0, 0, 0);
      }

      // weighted ReLU over this lane's 16 heads, then the other 16 from lane ^ 32
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p0 = __builtin_fmaf(wv[g][e], __builtin_fmaxf(acc0[4 * g + e], 0.f), p0);
          p1 = __builtin_fmaf(wv[g][e], __builtin_fmaxf(acc1[4 * g + e], 0.f), p1);
        }
      }
      p0 += __shfl_xor(p0, 32);
      p1 += __shfl_xor(p1, 32);
      // lane < 32 owns position lane of the first half, lane >= 32 position lane of the second
      val = half ? p1 : p0;
    }
    if (base + lane >= len) val = -__builtin_inff();  // partial last page
  }
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), out, lane * 4, 0, 0);
}

__global__ __launch_bounds__(256) void hwm_kernel(const int32_t* __restrict__ seq_lens, int32_t batch,
                                                   int32_t width, int32_t* __restrict__ row_hwm) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  const rsrc_t lens = make_rsrc(seq_lens, batch * sizeof(int32_t));
  const rsrc_t marks = make_rsrc(row_hwm, batch * sizeof(int32_t));
  if (b < batch) {
    const int len = (int)__builtin_amdgcn_raw_buffer_load_b32(lens, b * 4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32((uint32_t)clamp_len(len, width), marks, b * 4, 0, 0);
  }
}

}  // namespace

hipError_t launch_score(const void* q, const float* w, const void* k_pool, int64_t num_pages,
                        const int32_t* page_table, const int32_t* seq_lens, int32_t batch,
                        int32_t max_pages, float* logits, int32_t* row_hwm, hipStream_t stream) {
  hipLaunchKernelGGL(score_kernel, dim3(max_pages, batch), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(q), w, static_cast<const uint16_t*>(k_pool), num_pages,
                     page_table, seq_lens, max_pages, logits, row_hwm);
  if (row_hwm != nullptr) {
    // after every workgroup of the score kernel has read the old marks
    hipLaunchKernelGGL(hwm_kernel, dim3((batch + 255) / 256), dim3(256), 0, stream, seq_lens, batch,
                       max_pages * kPage, row_hwm);
  }
  return hipGetLastError();
}

}  // namespace dsa
