// Merge of two partial attention results over disjoint key sets.
//
// The passing block is the one input of the attention step that depends on the
// exchange between hosts (juejin.cn APB explainer, section "APB 的主要功能":
// compressed blocks are all-gathered into the passing block, then each host
// attends over anchor, passing and local blocks).  Attending over anchor + local
// first and over the passing block later gives two partial results (O_a, lse_a)
// and (O_b, lse_b); the softmax over the union of the key sets is
//   m = max(lse_a, lse_b),  w_x = exp(lse_x - m),
//   O = (w_a O_a + w_b O_b) / (w_a + w_b),  lse = m + ln(w_a + w_b),
// the same rescaling FlashAttention's online softmax applies between key tiles.
//
// gfx950 design: a pure HBM stream (read 2 x O and 2 x lse, write O and lse).
// A workgroup takes kRows consecutive query rows, all heads; a thread handles
// one 16-byte chunk (8 bf16) of one (row, head) per step, so a row's heads are
// read and written as one contiguous, fully coalesced run.  The d/8 threads of
// one (row, head) sit in one wave and read the same two lse values (one
// broadcast load each); the first of them writes the merged lse.  A workgroup
// takes two rows and a thread issues the loads of both before it computes either,
// so enough bytes are in flight per CU to cover HBM latency; the partial O are
// read once, with non-temporal loads.  Measured at a Llama-3.1-8B host block
// (403 MB): 79 us with the caches as the previous call left them, 74 us after an
// eviction (5.1-5.5 TB/s), against 100 / 89 us with 16 rows per workgroup
// walked one at a time.  No division except by powers of two.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 2;     // rows per workgroup
constexpr int kUnroll = 2;   // rows whose loads are in flight together

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;  // round to nearest even
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

// Merge factors of one (row, head) from its two lse values: O = ca O_a + cb O_b.
struct MergeW {
  float ca, cb, lse;
};
__device__ __forceinline__ MergeW merge_weights(float la, float lb) {
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.69314718055994531f;
  MergeW r{0.f, 0.f, -INFINITY};
  const float m = fmaxf(la, lb);
  if (m != -INFINITY) {  // at least one side saw a key
    const float wa = exp2f((la - m) * kLog2e);
    const float wb = exp2f((lb - m) * kLog2e);
    const float sum = wa + wb;
    const float inv = 1.f / sum;
    r.ca = wa * inv;
    r.cb = wb * inv;
    r.lse = m + log2f(sum) * kLn2;
  }
  return r;
}

__device__ __forceinline__ uint4 merge_chunk(const uint4 xa, const uint4 xb, float ca, float cb) {
  uint4 o;
  o.x = pack_bf16(ca * bf16_lo(xa.x) + cb * bf16_lo(xb.x), ca * bf16_hi(xa.x) + cb * bf16_hi(xb.x));
  o.y = pack_bf16(ca * bf16_lo(xa.y) + cb * bf16_lo(xb.y), ca * bf16_hi(xa.y) + cb * bf16_hi(xb.y));
  o.z = pack_bf16(ca * bf16_lo(xa.z) + cb * bf16_lo(xb.z), ca * bf16_hi(xa.z) + cb * bf16_hi(xb.z));
  o.w = pack_bf16(ca * bf16_lo(xa.w) + cb * bf16_lo(xb.w), ca * bf16_hi(xa.w) + cb * bf16_hi(xb.w));
  return o;
}

__global__ __launch_bounds__(kThreads) void merge_attention_kernel(const MergeArgs a) {
  const int cph_log2 = (a.d == 128) ? 4 : 3;      // 16-byte chunks per (row, head): d / 8
  const int per_row = a.Hq << cph_log2;            // chunks per row
  const int row0 = blockIdx.x * kRows;
  const int row_end = min(row0 + kRows, a.L);

  for (int c = threadIdx.x; c < per_row; c += kThreads) {
    const int head = c >> cph_log2;
    const bool lead = (c & ((1 << cph_log2) - 1)) == 0;  // writes the merged lse
    // kUnroll rows at a time: every load of the group is issued before any
    // arithmetic.
    for (int r0 = row0; r0 < row_end; r0 += kUnroll) {
      uint4 xa[kUnroll], xb[kUnroll];
      float la[kUnroll], lb[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int row = r0 + u;
        if (row < row_end) {
          const size_t li = (size_t)head * a.L + row;
          la[u] = a.la[li];
          lb[u] = a.lb[li];
          const size_t ci = (size_t)row * per_row + c;
          const u32x4 va = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.oa) + ci);
          const u32x4 vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.ob) + ci);
          xa[u] = uint4{va[0], va[1], va[2], va[3]};
          xb[u] = uint4{vb[0], vb[1], vb[2], vb[3]};
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int row = r0 + u;
        if (row < row_end) {
          const MergeW mw = merge_weights(la[u], lb[u]);
          reinterpret_cast<uint4 *>(a.out)[(size_t)row * per_row + c] =
              merge_chunk(xa[u], xb[u], mw.ca, mw.cb);
          if (a.lse != nullptr && lead) a.lse[(size_t)head * a.L + row] = mw.lse;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_merge_attention(const MergeArgs &a, hipStream_t s) {
  const int grid = (a.L + kRows - 1) / kRows;
  hipLaunchKernelGGL(merge_attention_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
