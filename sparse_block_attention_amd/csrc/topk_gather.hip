// APB step 2: keep the l best tokens per kv head and gather their K/V rows.
//
// juejin.cn APB explainer, section "APB 的主要功能": each host compresses its KV
// cache (keeps the important KV units) and the compressed blocks are sent to
// the other hosts.  Order: larger fp32 score first, -0 == +0, NaN below every
// number, ties to the lower token index; indices are written ascending.
//
// Selection is exact integer work on order-preserving 32-bit keys:
//  1. radix select, most significant digits first.  The leading bits shared by
//     the smallest and the largest key are shared by every key and are skipped;
//     the remaining bits go in digits of at most 12 bits (4096-bin LDS
//     histogram), so the first pass spreads the keys over their actual range.
//     Each pass keeps only the keys whose higher digits match the digits chosen
//     so far; a suffix scan over the bins (largest digit first) finds the digit
//     of the l-th best key.  The result is the key T of the l-th best element
//     and how many elements equal to T are still needed (`need`).  When the
//     chosen bin holds exactly the keys still needed, all of them are kept and
//     the lower digits are skipped: T is the bin's lowest key and every key
//     >= T is kept.
//  2. a stable compaction in index order keeps every key > T and the first
//     `need` keys == T.  With keys in LDS each thread owns a run of consecutive
//     indices and one block scan of its counts places its kept keys; above
//     that, each wave owns a contiguous run and ballots plus lane-mask bit
//     counts place them.  Either way the result does not depend on timing.
// gfx950 design: one 1024-thread workgroup (16 wave64s) per kv head.  Keys stay
// in LDS (128 KB) when the block has at most 32768 tokens; otherwise every pass
// re-reads the fp32 scores, which stay in L2 (512 KB per head at 131072
// tokens).  Scans are wave scans (cross-lane shuffles) plus one barrier for the
// 16 wave totals; starting the digits below the shared leading bits keeps the
// LDS histogram atomics from piling onto a few bins.
// The gather is a separate wide kernel: one workgroup per selected slot and
// tensor, 16 bytes per thread, contiguous rows.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kLdsKeys = 32768;
constexpr int kBins = 4096;

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;                       // NaN: below everything
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;                // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scan of v over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Batches of loads: every loop over the keys issues kBatch independent loads
// before it uses any, so a thread waits for one memory latency per batch rather
// than one per key.
constexpr int kBatch = 8;

template <bool KEYS_IN_LDS>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(const TopkArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[KEYS_IN_LDS ? kLdsKeys : 1];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wtot[2][kTopkWaves];
  __shared__ uint32_t sel_digit, sel_greater, sel_count;

  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = a.L;
  const float *srow = a.scores + (size_t)h * L;
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (KEYS_IN_LDS) return keys[i];
    else return order_key(srow[i]);
  };
  // f(i, key) for i = tid, tid + 1024, ... < L, in batches of kBatch loads
  auto for_each_key = [&](bool from_scores, auto &&f) {
    for (int base = 0; base < L; base += kBatch * kTopkThreads) {
      uint32_t kb[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        // clamped, so every load is in bounds and none waits behind a branch
        const int i = min(base + j * kTopkThreads + tid, L - 1);
        kb[j] = from_scores ? order_key(srow[i]) : key_at(i);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = base + j * kTopkThreads + tid;
        if (i < L) f(i, kb[j]);
      }
    }
  };
  // 0. keys into LDS (when they fit), and the bits every key shares: the common
  // leading bits of the smallest and the largest key.  They need no pass; the
  // first digit starts below them.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  bool loaded = false;
  if constexpr (KEYS_IN_LDS) {
    static_assert(kLdsKeys / 4 <= kBatch * kTopkThreads, "one batch of 16-byte loads");
    if ((L & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0) {
      // rows start 16-byte aligned: 16-byte loads, all of a thread's in one batch
      // (at most 32768 / 4 / 1024 = 8 per thread)
      const int n4 = L >> 2;
      const float4 *s4 = reinterpret_cast<const float4 *>(srow);
      float4 fb[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) fb[j] = s4[min(j * kTopkThreads + tid, n4 - 1)];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i4 = j * kTopkThreads + tid;
        if (i4 < n4) {
          const uint4 kq = make_uint4(order_key(fb[j].x), order_key(fb[j].y), order_key(fb[j].z),
                                      order_key(fb[j].w));
          *reinterpret_cast<uint4 *>(&keys[4 * i4]) = kq;
          kmin = min(kmin, min(min(kq.x, kq.y), min(kq.z, kq.w)));
          kmax = max(kmax, max(max(kq.x, kq.y), max(kq.z, kq.w)));
        }
      }
      loaded = true;
    }
  }
  if (!loaded) {
    for_each_key(true, [&](int i, uint32_t kk) {
      if constexpr (KEYS_IN_LDS) keys[i] = kk;
      kmin = min(kmin, kk);
      kmax = max(kmax, kk);
    });
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor(kmin, d, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor(kmax, d, 64));
  }
  if (lane == 0) {
    wtot[0][wave] = kmin;
    wtot[1][wave] = kmax;
  }
  __syncthreads();
  kmin = wtot[0][0];
  kmax = wtot[1][0];
  for (int w = 1; w < kTopkWaves; ++w) {
    kmin = min(kmin, wtot[0][w]);
    kmax = max(kmax, wtot[1][w]);
  }
  const int common = (kmin == kmax) ? 32 : __builtin_clz(kmin ^ kmax);  // shared leading bits
  __syncthreads();  // wtot is reused below

  // 1. radix select of the l-th largest key over the bits below the common
  // ones: digits of at most 12 bits, most significant first
  uint32_t prefix = common == 32 ? kmin : (common ? (kmin >> (32 - common)) << (32 - common) : 0u);
  uint32_t mask = common == 32 ? 0xffffffffu : (common ? ~0u << (32 - common) : 0u);
  int k_rem = a.l;
  int low = 32 - common;                        // bits still to resolve: [low-1 .. 0]
  bool take_all_eq = false;
#pragma unroll 1
  while (low > 0) {
    const int width = low < 12 ? low : 12;
    const int shift = low - width;
    const uint32_t dmask = (1u << width) - 1u;
    low = shift;
    for (int b = tid; b < kBins; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for_each_key(false, [&](int, uint32_t kk) {
      if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & dmask], 1u);
    });
    __syncthreads();
    // Thread t holds bins 4095-4t .. 4092-4t (largest digit first); the scan over
    // threads gives #candidates with digit >= each thread's last bin.
    uint32_t c[4];
    uint32_t s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = hist[kBins - 1 - (4 * tid + j)];
      s += c[j];
    }
    const uint32_t incl_w = wave_inclusive_scan(s, lane);
    if (lane == 63) wtot[0][wave] = incl_w;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[0][w];
    const uint32_t incl = base + incl_w;
    const uint32_t excl = incl - s;
    if (excl < (uint32_t)k_rem && incl >= (uint32_t)k_rem) {  // exactly one thread
      uint32_t acc = excl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (acc + c[j] >= (uint32_t)k_rem) {
          sel_digit = (uint32_t)(kBins - 1 - (4 * tid + j));
          sel_greater = acc;
          sel_count = c[j];
          break;
        }
        acc += c[j];
      }
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= dmask << shift;
    k_rem -= (int)sel_greater;
    // Every key of the chosen bin is kept when the bin holds exactly the keys still
    // needed: then the kept set is {key >= prefix} whatever the lower bits, and the
    // remaining digits are skipped (prefix has zeros below the resolved bits).
    if (sel_count == (uint32_t)k_rem) {
      take_all_eq = true;
      break;
    }
  }
  const uint32_t T = prefix;
  // elements == T to keep, >= 1 (all of them after an early exit: keys > T and == T
  // are then both kept, at positions counting both)
  const uint32_t need = take_all_eq ? 0xffffffffu : (uint32_t)k_rem;

  // (common == 32: every key equals kmin, which is T)
  int32_t *out = a.idx + (size_t)h * a.l;
  const uint32_t l = (uint32_t)a.l;
  if constexpr (KEYS_IN_LDS) {
    // 2. stable compaction, keys in LDS: thread t owns the run of `per` consecutive
    // indices starting at t*per (per a multiple of 4, so each run is read with
    // 16-byte loads into registers); one block-wide scan of the per-thread counts
    // of keys > T and == T gives every thread its output positions.
    constexpr int kMaxPer = kLdsKeys / kTopkThreads;   // 32
    const int per = (((L + kTopkThreads - 1) / kTopkThreads) + 3) & ~3;
    const int b = tid * per;
    uint32_t kr[kMaxPer];
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kMaxPer; j += 4) {
      if (j < per) {
        const uint4 q4 = *reinterpret_cast<const uint4 *>(&keys[b + j]);
        kr[j] = q4.x;
        kr[j + 1] = q4.y;
        kr[j + 2] = q4.z;
        kr[j + 3] = q4.w;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool in = b + j + u < L;
          ngt += (in && kr[j + u] > T) ? 1u : 0u;
          neq += (in && kr[j + u] == T) ? 1u : 0u;
        }
      }
    }
    const uint32_t ig = wave_inclusive_scan(ngt, lane);
    const uint32_t ie = wave_inclusive_scan(neq, lane);
    if (lane == 63) {
      wtot[0][wave] = ig;
      wtot[1][wave] = ie;
    }
    __syncthreads();
    uint32_t g = ig - ngt, e = ie - neq;            // keys > T and == T before this run
    for (int w = 0; w < wave; ++w) {
      g += wtot[0][w];
      e += wtot[1][w];
    }
#pragma unroll
    for (int j = 0; j < kMaxPer; ++j) {
      if (j < per && b + j < L) {
        const uint32_t kk = kr[j];
        if (kk > T) {
          const uint32_t pos = g + min(e, need);
          if (pos < l) out[pos] = b + j;
          ++g;
        } else if (kk == T) {
          if (e < need && g + e < l) out[g + e] = b + j;
          ++e;
        }
      }
    }
    return;
  }
  // 2. stable compaction: wave w owns indices [w*C, (w+1)*C), C a multiple of 64
  const int C = ((L + kTopkThreads - 1) / kTopkThreads) * 64;
  const int lo = min(wave * C, L);
  const int hi = min(lo + C, L);
  // f(i, key, valid) over this wave's run, 64 consecutive indices per step, in
  // batches of kBatch steps
  auto for_each_run_key = [&](auto &&f) {
    for (int b0 = lo; b0 < hi; b0 += 64 * kBatch) {
      uint32_t kb[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) kb[j] = key_at(min(b0 + 64 * j + lane, hi - 1));
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = b0 + 64 * j + lane;
        if (b0 + 64 * j < hi) f(i, kb[j], i < hi);   // wave-uniform step condition
      }
    }
  };
  uint32_t ngt = 0, neq = 0;
  for_each_run_key([&](int, uint32_t kk, bool valid) {
    ngt += __popcll(__ballot(valid && kk > T));
    neq += __popcll(__ballot(valid && kk == T));
  });
  if (lane == 0) {
    wtot[0][wave] = ngt;
    wtot[1][wave] = neq;
  }
  __syncthreads();
  uint32_t g_before = 0, e_before = 0;
  for (int w = 0; w < wave; ++w) {
    g_before += wtot[0][w];
    e_before += wtot[1][w];
  }
  for_each_run_key([&](int i, uint32_t kk, bool valid) {
    const bool gt = valid && kk > T;
    const bool eq = valid && kk == T;
    const unsigned long long bg = __ballot(gt);
    const unsigned long long be = __ballot(eq);
    const uint32_t g = g_before + lanes_below(bg);
    const uint32_t e = e_before + lanes_below(be);
    if (gt) {
      const uint32_t pos = g + min(e, need);
      if (pos < l) out[pos] = i;
    } else if (eq && e < need) {
      const uint32_t pos = g + e;
      if (pos < l) out[pos] = i;
    }
    g_before += __popcll(bg);
    e_before += __popcll(be);
  });
}

// One workgroup per (slot s, tensor): copies row idx[h][s] of every kv head h.
__global__ __launch_bounds__(128) void gather_kernel(const TopkArgs a) {
  const int s = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int ch_log2 = (a.d == 128) ? 4 : 3;     // 16-byte chunks per head row: d / 8
  const int n = a.Hkv << ch_log2;               // chunks in one [Hkv][d] row
  const uint16_t *src_base = is_v ? a.v : a.k;
  uint16_t *dst = (is_v ? a.vc : a.kc) + (size_t)s * n * 8;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    const int hh = j >> ch_log2;
    const int c = j & ((1 << ch_log2) - 1);
    int tok = a.idx[(size_t)hh * a.l + s];
    if ((unsigned)tok >= (unsigned)a.L) tok = 0;  // never read outside the block
    const uint16_t *src = src_base + ((size_t)tok * a.Hkv + hh) * a.d + c * 8;
    reinterpret_cast<uint4 *>(dst)[j] = *reinterpret_cast<const uint4 *>(src);
  }
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
  hipLaunchKernelGGL(gather_kernel, dim3(a.l, 2), dim3(128), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
