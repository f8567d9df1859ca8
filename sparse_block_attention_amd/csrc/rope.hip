// Rotary position embedding (rotate-half pairing) on token-major [rows][heads][d].
//
// Before the attention steps: the Llama models the pages evaluate on encode
// positions by rotating each (i, i + d/2) pair of q and k by the angle
// position * theta_i, theta_i = base^(-2i/d) (the Llama 3 paper is among the
// works the mlsanity.com APB page lists).
//
// gfx950 design: a pure HBM stream (read and write d*2 bytes per head row).  A
// thread takes one token row, 8 consecutive pairs (16 bytes from each half of a
// head row) and every fourth head of the row: it forms its 8 angles once and walks
// its heads four at a time, all loads issued first (non-temporal: each input byte
// is read once).  The d/16 threads of a row and head sit side by side, so each
// head row is read and written as whole 128-byte pieces.  Four threads share a
// row's angles (each forms them) so that four times as many waves keep loads in
// flight.  q and k of a Llama-3.1-8B host block, 336 MB, back to back: 86 us with
// one workgroup per row and 8-byte accesses, 75 us with one thread per (row,
// pairs) walking all heads, 68 us now.
// The angle pos * theta_i is formed and reduced modulo 2*pi in double precision
// (Cody-Waite with a two-part 2*pi): with positions below 2^31 the reduced angle
// is within about 2^-21 rad of the exact one; sin/cos and the rotation run in
// fp32 and each output is rounded once to bf16.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeSplitLog2 = 2;                 // threads per (row, pairs): 4
constexpr int kRopeSplit = 1 << kRopeSplitLog2;   // each takes every fourth head
constexpr int kRopeUnroll = 4;                    // heads whose loads are in flight together
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

// x0' = x0 cos - x1 sin, x1' = x0 sin + x1 cos for the 8 pairs of one 16-byte
// piece of each half.
__device__ __forceinline__ void rotate8(const uint4 lo, const uint4 hi, const float (&c)[8], const float (&s)[8],
                                        uint4 &olo, uint4 &ohi) {
  const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w};
  const uint32_t h[4] = {hi.x, hi.y, hi.z, hi.w};
  uint32_t ol[4], oh[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = bf16_lo(l[w]), a1 = bf16_hi(l[w]);  // pairs 2w, 2w+1: first half
    const float b0 = bf16_lo(h[w]), b1 = bf16_hi(h[w]);  // second half
    ol[w] = pack_bf16(a0 * c[2 * w] - b0 * s[2 * w], a1 * c[2 * w + 1] - b1 * s[2 * w + 1]);
    oh[w] = pack_bf16(a0 * s[2 * w] + b0 * c[2 * w], a1 * s[2 * w + 1] + b1 * c[2 * w + 1]);
  }
  olo = uint4{ol[0], ol[1], ol[2], ol[3]};
  ohi = uint4{oh[0], oh[1], oh[2], oh[3]};
}

__global__ __launch_bounds__(kRopeThreads) void rope_kernel(const RopeArgs a) {
  const int jpr_log2 = (a.d == 128) ? 3 : 2;          // 8-pair pieces per half row: d / 16
  const int tpr_log2 = jpr_log2 + kRopeSplitLog2;     // threads per row
  const int rows_per_wg = kRopeThreads >> tpr_log2;
  const int j = threadIdx.x & ((1 << jpr_log2) - 1);  // this thread's pairs: 8j .. 8j+7
  const int hs = (threadIdx.x >> jpr_log2) & (kRopeSplit - 1);  // heads hs, hs + 4, ...
  const int row = blockIdx.x * rows_per_wg + (threadIdx.x >> tpr_log2);
  if (row >= a.rows) return;
  const int half_d = a.d >> 1;
  const double pos = (double)(a.pos0 + row);
  constexpr double kTwoPiHi = 6.283185307179586232;   // 2*pi = hi + lo
  constexpr double kTwoPiLo = 2.449293598294706e-16;
  constexpr double kInvTwoPi = 0.15915494309189535;
  float c[8], s[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const double ang = pos * a.theta[8 * j + u];
    const double n = rint(ang * kInvTwoPi);
    const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, ang));
    sincosf((float)r, &s[u], &c[u]);
  }
  const uint16_t *xr = a.x + (size_t)row * a.heads * a.d + 8 * j;
  uint16_t *orow = a.out + (size_t)row * a.heads * a.d + 8 * j;
  for (int h0 = hs; h0 < a.heads; h0 += kRopeSplit * kRopeUnroll) {
    uint4 lo[kRopeUnroll], hi[kRopeUnroll];
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      const int h = h0 + kRopeSplit * u;
      if (h < a.heads) {
        const u32x4 vl = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)h * a.d));
        const u32x4 vh = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xr + (size_t)h * a.d + half_d));
        lo[u] = uint4{vl[0], vl[1], vl[2], vl[3]};
        hi[u] = uint4{vh[0], vh[1], vh[2], vh[3]};
      }
    }
#pragma unroll
    for (int u = 0; u < kRopeUnroll; ++u) {
      const int h = h0 + kRopeSplit * u;
      if (h < a.heads) {
        uint4 olo, ohi;
        rotate8(lo[u], hi[u], c, s, olo, ohi);
        *reinterpret_cast<uint4 *>(orow + (size_t)h * a.d) = olo;
        *reinterpret_cast<uint4 *>(orow + (size_t)h * a.d + half_d) = ohi;
      }
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, hipStream_t s) {
  const int rows_per_wg = kRopeThreads / (a.d / 16) / kRopeSplit;
  hipLaunchKernelGGL(rope_kernel, dim3((a.rows + rows_per_wg - 1) / rows_per_wg), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
