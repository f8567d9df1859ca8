// Rotary position embedding (rotate-half pairing) on token-major [rows][heads][d].
//
// Before the attention steps: the Llama models the pages evaluate on encode
// positions by rotating each (i, i + d/2) pair of q and k by the angle
// position * theta_i, theta_i = base^(-2i/d) (the Llama 3 paper is among the
// works the mlsanity.com APB page lists).
//
// gfx950 design: a pure HBM stream (read and write d*2 bytes per head row).  A
// workgroup takes one token row; a thread handles 4 consecutive pairs (8 bytes
// from each half of a head row) and keeps their (cos, sin) for every head of
// the row, since the angle depends on the position and i only.  The angle
// pos * theta_i is formed and reduced modulo 2*pi in double precision
// (Cody-Waite with a two-part 2*pi): with positions below 2^31 the reduced angle
// is within about 2^-21 rad of the exact one; sin/cos and the rotation run in
// fp32 and each output is rounded once to bf16.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kRopeThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

__global__ __launch_bounds__(kRopeThreads) void rope_kernel(const RopeArgs a) {
  const int row = blockIdx.x;
  const int half_d = a.d >> 1;
  const int cpr_log2 = (a.d == 128) ? 4 : 3;        // 4-pair chunks per head row: d / 8
  const int j = threadIdx.x & ((1 << cpr_log2) - 1); // this thread's chunk: pairs 4j .. 4j+3
  const double pos = (double)(a.pos0 + row);
  constexpr double kTwoPiHi = 6.283185307179586232;   // 2*pi = hi + lo
  constexpr double kTwoPiLo = 2.449293598294706e-16;
  constexpr double kInvTwoPi = 0.15915494309189535;
  float c[4], s[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const double ang = pos * a.theta[4 * j + u];
    const double n = rint(ang * kInvTwoPi);
    const double r = fma(-n, kTwoPiLo, fma(-n, kTwoPiHi, ang));
    sincosf((float)r, &s[u], &c[u]);
  }
  const size_t row_base = (size_t)row * a.heads * a.d;
  const int n_chunks = a.heads << cpr_log2;
  for (int cidx = threadIdx.x; cidx < n_chunks; cidx += kRopeThreads) {
    const int h = cidx >> cpr_log2;
    const size_t lo_off = row_base + (size_t)h * a.d + 4 * j;
    const uint2 xl = *reinterpret_cast<const uint2 *>(a.x + lo_off);
    const uint2 xh = *reinterpret_cast<const uint2 *>(a.x + lo_off + half_d);
    const uint16_t *pl = reinterpret_cast<const uint16_t *>(&xl);
    const uint16_t *ph = reinterpret_cast<const uint16_t *>(&xh);
    uint16_t ol[4], oh[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x0 = bf16_to_f32(pl[u]);
      const float x1 = bf16_to_f32(ph[u]);
      ol[u] = f32_to_bf16(x0 * c[u] - x1 * s[u]);
      oh[u] = f32_to_bf16(x0 * s[u] + x1 * c[u]);
    }
    *reinterpret_cast<uint2 *>(a.out + lo_off) = *reinterpret_cast<const uint2 *>(ol);
    *reinterpret_cast<uint2 *>(a.out + lo_off + half_d) = *reinterpret_cast<const uint2 *>(oh);
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(rope_kernel, dim3(a.rows), dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
