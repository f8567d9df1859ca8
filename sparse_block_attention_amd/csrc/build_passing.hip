// APB step 3: passing block from the compressed blocks of the preceding hosts.
//
// juejin.cn APB explainer, section "APB 的主要功能": the compressed blocks are
// all-gathered and form the passing block, which carries the important KV of
// the preceding hosts; section "APB 的技术原理": each context block is
// compressed and sent on to the later GPUs.  Layout: host-major, row j*l + s
// holds slot s of host j, so host j's block is one contiguous run.
//
// One launch copies up to 128 source blocks for K and V: grid.y enumerates
// (source, tensor) pairs, grid.x strides over 16-byte units with 4 units in
// flight per thread.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void build_passing_kernel(const PassArgs a) {
  const int src_i = blockIdx.y >> 1;
  const bool is_v = blockIdx.y & 1;
  const uint4 *src = reinterpret_cast<const uint4 *>(is_v ? a.vsrc[src_i] : a.ksrc[src_i]);
  uint4 *dst = reinterpret_cast<uint4 *>(is_v ? a.vdst : a.kdst) + (long long)src_i * a.block_u16x8;
  const long long n = a.block_u16x8;
  const long long step = (long long)gridDim.x * kThreads * kUnroll;
  for (long long base = (long long)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n; base += step) {
    if (base + (kUnroll - 1) * kThreads < n) {
      const uint4 r0 = src[base];
      const uint4 r1 = src[base + kThreads];
      const uint4 r2 = src[base + 2 * kThreads];
      const uint4 r3 = src[base + 3 * kThreads];
      dst[base] = r0;
      dst[base + kThreads] = r1;
      dst[base + 2 * kThreads] = r2;
      dst[base + 3 * kThreads] = r3;
    } else {
      for (long long i = base; i < n; i += kThreads) dst[i] = src[i];
    }
  }
}

}  // namespace

hipError_t launch_build_passing(const PassArgs &a, hipStream_t s) {
  const long long per_block = (long long)kThreads * kUnroll;
  long long gx = (a.block_u16x8 + per_block - 1) / per_block;
  if (gx > 1024) gx = 1024;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(build_passing_kernel, dim3((unsigned)gx, 2 * a.n_src), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
