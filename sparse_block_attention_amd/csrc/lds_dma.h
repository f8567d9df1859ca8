// LDS-DMA building blocks shared by the streaming MFMA kernels (scorer and
// projection): chunk rows go HBM -> LDS with buffer_load ... lds, 1 KB per
// instruction.  Device code for gfx950; included by .hip sources only.
#pragma once

#include "apb_internal.h"

namespace apb {

typedef __attribute__((address_space(3))) void lds_void;

// One 1 KB LDS-DMA load (64 lanes x 16 bytes).  Base and range are the same in
// every lane; readfirstlane says so, so the descriptor lives in scalar registers.
// (Device pass only: the host pass has no buffer-descriptor type.)
__device__ __forceinline__ void dma_1k(const void *base, int valid_bytes, int voff, uint8_t *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void *>(ub), 0, __builtin_amdgcn_readfirstlane(valid_bytes), 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, voff, 0, 0, 0);
#endif
}

// s_waitcnt vmcnt(n) for a wave-uniform n known only at run time (n <= 23;
// larger n waits for everything, which is always safe).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  switch (n) {
#define APB_CASE(N) \
  case N: wait_vmcnt<N>(); break;
    APB_CASE(1) APB_CASE(2) APB_CASE(3) APB_CASE(4) APB_CASE(5) APB_CASE(6) APB_CASE(7) APB_CASE(8)
    APB_CASE(9) APB_CASE(10) APB_CASE(11) APB_CASE(12) APB_CASE(13) APB_CASE(14) APB_CASE(15)
    APB_CASE(16) APB_CASE(17) APB_CASE(18) APB_CASE(19) APB_CASE(20) APB_CASE(21) APB_CASE(22)
    APB_CASE(23)
#undef APB_CASE
    default: wait_vmcnt<0>(); break;
  }
}

}  // namespace apb
