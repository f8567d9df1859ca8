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
// broadcast load each); the first of them writes the merged lse.  kRows = 16
// consecutive rows make each 64-byte lse line be used whole.  No division
// except by powers of two.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;  // round to nearest even
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

__global__ __launch_bounds__(kThreads) void merge_attention_kernel(const MergeArgs a) {
  const int cph_log2 = (a.d == 128) ? 4 : 3;      // 16-byte chunks per (row, head): d / 8
  const int per_row = a.Hq << cph_log2;            // chunks per row
  const int row0 = blockIdx.x * kRows;
  const int row_end = min(row0 + kRows, a.L);
  constexpr float kLog2e = 1.4426950408889634f;
  constexpr float kLn2 = 0.69314718055994531f;

  for (int row = row0; row < row_end; ++row) {
    const size_t rbase = (size_t)row * per_row;
    for (int c = threadIdx.x; c < per_row; c += kThreads) {
      const int head = c >> cph_log2;
      const size_t li = (size_t)head * a.L + row;
      const float la = a.la[li], lb = a.lb[li];
      const float m = fmaxf(la, lb);
      float wa = 0.f, wb = 0.f, inv = 0.f, lse = -INFINITY;
      if (m != -INFINITY) {  // at least one side saw a key
        wa = exp2f((la - m) * kLog2e);
        wb = exp2f((lb - m) * kLog2e);
        const float sum = wa + wb;
        inv = 1.f / sum;
        lse = m + log2f(sum) * kLn2;
      }
      const uint4 xa = reinterpret_cast<const uint4 *>(a.oa)[rbase + c];
      const uint4 xb = reinterpret_cast<const uint4 *>(a.ob)[rbase + c];
      const float ca = wa * inv, cb = wb * inv;
      uint4 o;
      o.x = pack_bf16(ca * bf16_lo(xa.x) + cb * bf16_lo(xb.x), ca * bf16_hi(xa.x) + cb * bf16_hi(xb.x));
      o.y = pack_bf16(ca * bf16_lo(xa.y) + cb * bf16_lo(xb.y), ca * bf16_hi(xa.y) + cb * bf16_hi(xb.y));
      o.z = pack_bf16(ca * bf16_lo(xa.z) + cb * bf16_lo(xb.z), ca * bf16_hi(xa.z) + cb * bf16_hi(xb.z));
      o.w = pack_bf16(ca * bf16_lo(xa.w) + cb * bf16_lo(xb.w), ca * bf16_hi(xa.w) + cb * bf16_hi(xb.w));
      reinterpret_cast<uint4 *>(a.out)[rbase + c] = o;
      if (a.lse != nullptr && (c & ((1 << cph_log2) - 1)) == 0) a.lse[li] = lse;
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
