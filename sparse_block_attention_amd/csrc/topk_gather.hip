// APB step 2: keep the l best tokens per kv head and gather their K/V rows.
//
// juejin.cn APB explainer, section "APB 的主要功能": each host compresses its KV
// cache (keeps the important KV units) and the compressed blocks are sent to
// the other hosts.  Order: larger fp32 score first, -0 == +0, NaN below every
// number, ties to the lower token index; indices are written ascending.
//
// Selection is exact integer work on order-preserving 32-bit keys:
//  1. radix select, most significant byte first (4 passes of a 256-bin LDS
//     histogram), finds the key T of the l-th best element and how many
//     elements equal to T are still needed (`need`);
//  2. one stable compaction in index order keeps every key > T and the first
//     `need` keys == T.  A block scan of (count > T, count == T) pairs gives each
//     thread its output position, so the result does not depend on timing.
// One 1024-thread workgroup per kv head; keys stay in LDS when the block has at
// most 16384 tokens, otherwise each pass re-reads the (L2-resident) scores.
// The gather is a separate wide kernel: 16 bytes per thread, coalesced rows.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kLdsKeys = 16384;

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;                       // NaN: below everything
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;                // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive Hillis-Steele scan over n <= blockDim.x entries of buf (in place).
template <typename T>
__device__ void block_inclusive_scan(T *buf, int n) {
  const int tid = threadIdx.x;
  for (int off = 1; off < n; off <<= 1) {
    T add = 0;
    if (tid < n && tid >= off) add = buf[tid - off];
    __syncthreads();
    if (tid < n) buf[tid] += add;
    __syncthreads();
  }
}

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(const TopkArgs a) {
  __shared__ uint32_t keys[KEYS_IN_LDS ? kLdsKeys : 1];
  __shared__ uint32_t hist[256];
  __shared__ unsigned long long scan[kTopkThreads];
  __shared__ uint32_t sel_digit, sel_greater;

  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = a.L;
  const float *srow = a.scores + (size_t)h * L;
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (KEYS_IN_LDS) return keys[i];
    else return order_key(srow[i]);
  };
  if constexpr (KEYS_IN_LDS) {
    for (int i = tid; i < L; i += kTopkThreads) keys[i] = order_key(srow[i]);
    __syncthreads();
  }

  // 1. radix select of the l-th largest key
  uint32_t prefix = 0, mask = 0;
  int k_rem = a.l;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < L; i += kTopkThreads) {
      const uint32_t kk = key_at(i);
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix sums: scan[t] = #candidates with digit >= 255 - t
    if (tid < 256) scan[tid] = hist[255 - tid];
    __syncthreads();
    block_inclusive_scan(scan, 256);
    if (tid < 256) {
      const unsigned long long ge = scan[tid];                   // digit >= 255 - tid
      const unsigned long long gt = tid ? scan[tid - 1] : 0ull;  // digit >  255 - tid
      if (ge >= (unsigned long long)k_rem && gt < (unsigned long long)k_rem) {
        sel_digit = 255 - tid;
        sel_greater = (uint32_t)gt;
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    k_rem -= (int)sel_greater;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const unsigned need = (unsigned)k_rem;       // elements == T to keep, >= 1

  // 2. stable compaction in index order
  const int per = (L + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(tid * per, L);
  const int hi = min(lo + per, L);
  unsigned n_gt = 0, n_eq = 0;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key_at(i);
    n_gt += kk > T;
    n_eq += kk == T;
  }
  scan[tid] = ((unsigned long long)n_eq << 32) | n_gt;
  __syncthreads();
  block_inclusive_scan(scan, kTopkThreads);
  const unsigned long long excl = tid ? scan[tid - 1] : 0ull;
  unsigned g_before = (unsigned)(excl & 0xffffffffull);
  unsigned e_before = (unsigned)(excl >> 32);
  int32_t *out = a.idx + (size_t)h * a.l;
  for (int i = lo; i < hi; ++i) {
    const uint32_t kk = key_at(i);
    if (kk > T) {
      const unsigned pos = g_before + min(e_before, need);
      if (pos < (unsigned)a.l) out[pos] = i;
      ++g_before;
    } else if (kk == T) {
      if (e_before < need && g_before + e_before < (unsigned)a.l) out[g_before + e_before] = i;
      ++e_before;
    }
  }
}

__global__ __launch_bounds__(256) void gather_kernel(const TopkArgs a) {
  const int ch = a.d / 8;
  const long long rows = (long long)a.l * a.Hkv;
  const long long total = 2 * rows * ch;
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int c = (int)(t % ch);
  const long long r = t / ch;
  const bool is_v = r >= rows;
  const long long rr = is_v ? r - rows : r;
  const int s = (int)(rr / a.Hkv);
  const int hh = (int)(rr % a.Hkv);
  int tok = a.idx[(size_t)hh * a.l + s];
  if ((unsigned)tok >= (unsigned)a.L) tok = 0;  // never read outside the block
  const uint16_t *src = (is_v ? a.v : a.k) + ((size_t)tok * a.Hkv + hh) * a.d + c * 8;
  uint16_t *dst = (is_v ? a.vc : a.kc) + ((size_t)s * a.Hkv + hh) * a.d + c * 8;
  *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
}

}  // namespace

hipError_t launch_topk_gather(const TopkArgs &a, hipStream_t s) {
  if (a.L <= kLdsKeys) {
    hipLaunchKernelGGL((topk_select_kernel<true>), dim3(a.Hkv), dim3(kTopkThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((topk_select_kernel<false>), dim3(a.Hkv), dim3(kTopkThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long total = 2LL * a.l * a.Hkv * (a.d / 8);
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
