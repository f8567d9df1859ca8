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
//  2. per-chunk counts: for every chunk of 256 keys, the number of keys > T and
//     == T in the chunks before it (an exclusive scan over the chunks).
//  3. compaction and gather: a wide kernel, one workgroup per chunk, keeps every
//     key > T and the first `need` keys == T in index order.  A kept key's slot
//     is the number of kept keys before it, from its chunk's counts and wave
//     ballots inside the chunk, so the result does not depend on timing; the
//     same workgroup then copies the kept keys' K and V head rows.
// gfx950 design: the select runs one 1024-thread workgroup (16 wave64s) per kv
// head.  Keys stay in LDS (128 KB) when the block has at most 32768 tokens;
// otherwise every pass re-reads the fp32 scores, which stay in L2 (512 KB per
// head at 131072 tokens).  Scans are wave scans (cross-lane shuffles) plus one
// barrier for the 16 wave totals; starting the digits below the shared leading
// bits keeps the LDS histogram atomics from piling onto a few bins.  The select
// hands T, `need` and the chunk counts to the placement kernel through the
// caller's workspace; every workspace word a call reads was written earlier in
// that call.  The placement kernel spreads the compaction and the 16-byte row
// copies over L/256 x Hkv workgroups.
#include <mutex>

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

// Sum of v over the 64 lanes of a wave, in every lane, with DPP moves: shifts by
// 1, 2, 4 and 8 lanes inside each row of 16 (lanes whose source lies outside the
// row add 0), lane 15 of each row added to the next row, lane 31 to the upper two
// rows, then lane 63 read.
__device__ __forceinline__ uint32_t wave_sum_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Batches of loads: every loop over the keys issues kBatch independent loads
// before it uses any, so a thread waits for one memory latency per batch rather
// than one per key.
constexpr int kBatch = 8;

// Placement chunk (keys per workgroup of the placement kernel) and the run of
// consecutive keys one thread of the select kernel counts per step.
constexpr int kChunk = 256;
constexpr int kRun = 16;

// Keys r*kRun .. r*kRun+kRun-1 of one head (entries past L are unspecified): from
// LDS when the keys are there, else from the fp32 scores, with 16-byte loads when
// the row allows them.
template <bool KEYS_IN_LDS>
__device__ __forceinline__ void load_run(const TopkArgs &a, const float *srow, const uint32_t *keys, int r,
                                         uint32_t (&kr)[kRun]) {
  const int b = r * kRun;
  if constexpr (KEYS_IN_LDS) {
#pragma unroll
    for (int j = 0; j < kRun; j += 4) {
      const uint4 q4 = *reinterpret_cast<const uint4 *>(&keys[b + j]);
      kr[j] = q4.x;
      kr[j + 1] = q4.y;
      kr[j + 2] = q4.z;
      kr[j + 3] = q4.w;
    }
  } else {
    if ((a.L & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0) {
      const int n4 = a.L >> 2;
      const float4 *s4 = reinterpret_cast<const float4 *>(srow);
      float4 f[kRun / 4];
#pragma unroll
      for (int j = 0; j < kRun / 4; ++j) f[j] = s4[min(b / 4 + j, n4 - 1)];
#pragma unroll
      for (int j = 0; j < kRun / 4; ++j) {
        kr[4 * j] = order_key(f[j].x);
        kr[4 * j + 1] = order_key(f[j].y);
        kr[4 * j + 2] = order_key(f[j].z);
        kr[4 * j + 3] = order_key(f[j].w);
      }
    } else {
      float f[kRun];
#pragma unroll
      for (int j = 0; j < kRun; ++j) f[j] = srow[min(b + j, a.L - 1)];
#pragma unroll
      for (int j = 0; j < kRun; ++j) kr[j] = order_key(f[j]);
    }
  }
}

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
  // Rows whose fp32 scores start 16-byte aligned are read with 16-byte loads.
  const bool vec = (L & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
  // f(i, key) for every key i < L, in batches of kBatch loads: from LDS (i = tid,
  // tid + 1024, ...), or from the scores, 16-byte blocks when the row allows (block
  // j of 4096 keys: thread t takes keys 4(j*1024 + t) .. +3).
  auto for_each_key = [&](bool from_scores, auto &&f) {
    if (!KEYS_IN_LDS && vec) {
      const int n4 = L >> 2;
      const float4 *s4 = reinterpret_cast<const float4 *>(srow);
      for (int base4 = 0; base4 < n4; base4 += kBatch * kTopkThreads) {
        float4 fb[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) fb[j] = s4[min(base4 + j * kTopkThreads + tid, n4 - 1)];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int q = base4 + j * kTopkThreads + tid;
          if (q < n4) {
            f(4 * q, order_key(fb[j].x));
            f(4 * q + 1, order_key(fb[j].y));
            f(4 * q + 2, order_key(fb[j].z));
            f(4 * q + 3, order_key(fb[j].w));
          }
        }
      }
      return;
    }
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
  // (common == 32: every key equals kmin, which is T)
  const uint32_t need = take_all_eq ? 0xffffffffu : (uint32_t)k_rem;

  // 2. per-chunk counts for the placement kernel: chunk c holds keys
  // [c*kChunk, (c+1)*kChunk); the workspace gets, for every chunk, the number of
  // keys > T and == T in the chunks before it.  A run of 16 consecutive keys is
  // counted by one thread, so the 16 runs of a chunk are 16 adjacent lanes of one
  // wave; groups of 1024 chunks are scanned in LDS (hist is free again) with a
  // running carry.
  // Keys read from the scores with 16-byte loads are counted by blocks instead: a
  // wave's share of a 4096-key block is one chunk, and a wave sum (DPP) counts it.
  static_assert(kChunk == 16 * kRun, "a chunk is 16 runs of adjacent lanes");
  static_assert(kChunk * kTopkWaves == 4 * kTopkThreads, "a chunk is one wave's share of a key block");
  uint32_t *cnt = a.chunk_counts + (size_t)h * a.n_chunks * 2;
  const int n_runs = (L + kRun - 1) / kRun;
  const bool by_blocks = !KEYS_IN_LDS && vec;
  uint32_t carry_gt = 0, carry_eq = 0;
#pragma unroll 1
  for (int c0 = 0; c0 < a.n_chunks; c0 += kTopkThreads) {
    if (by_blocks) {
      // chunks c0 .. c0+1023 are the wave shares of key blocks c0/16 .. c0/16+63
      const int n4 = L >> 2;
      const float4 *s4 = reinterpret_cast<const float4 *>(srow);
      const int jb0 = c0 / kTopkWaves;
      const int jb1 = min(jb0 + kTopkThreads / kTopkWaves, (n4 + kTopkThreads - 1) / kTopkThreads);
#pragma unroll 1
      for (int j0 = jb0; j0 < jb1; j0 += kBatch) {   // wave-uniform bounds
        float4 fb[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) fb[j] = s4[min((j0 + j) * kTopkThreads + tid, n4 - 1)];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          if (j0 + j < jb1) {   // wave-uniform
            const int q = (j0 + j) * kTopkThreads + tid;
            const uint32_t k4[4] = {order_key(fb[j].x), order_key(fb[j].y), order_key(fb[j].z), order_key(fb[j].w)};
            uint32_t ngt = 0, neq = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bool in = 4 * q + u < L;
              ngt += (in && k4[u] > T) ? 1u : 0u;
              neq += (in && k4[u] == T) ? 1u : 0u;
            }
            const uint32_t packed = wave_sum_dpp((ngt << 16) | neq);   // each count <= 256
            const int c = (j0 + j) * kTopkWaves + wave - c0;
            if (lane == 0 && c0 + c < a.n_chunks) {
              hist[c] = packed >> 16;
              hist[kTopkThreads + c] = packed & 0xffffu;
            }
          }
        }
      }
    }
#pragma unroll 1
    for (int rb = c0 * 16; !by_blocks && rb < min(n_runs, (c0 + kTopkThreads) * 16); rb += kTopkThreads) {
      const int r = rb + tid;
      uint32_t ngt = 0, neq = 0;
      if (r < n_runs) {
        uint32_t kr[kRun];
        load_run<KEYS_IN_LDS>(a, srow, keys, r, kr);
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
          const bool in = r * kRun + u < L;
          ngt += (in && kr[u] > T) ? 1u : 0u;
          neq += (in && kr[u] == T) ? 1u : 0u;
        }
      }
      uint32_t packed = (ngt << 16) | neq;            // each count <= 256
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) packed += (uint32_t)__shfl_xor((int)packed, m, 64);
      if ((lane & 15) == 0 && r < n_runs) {
        const int c = r / 16 - c0;
        hist[c] = packed >> 16;
        hist[kTopkThreads + c] = packed & 0xffffu;
      }
    }
    __syncthreads();
    const int c = c0 + tid;
    const uint32_t vg = c < a.n_chunks ? hist[tid] : 0u;
    const uint32_t ve = c < a.n_chunks ? hist[kTopkThreads + tid] : 0u;
    const uint32_t ig = wave_inclusive_scan(vg, lane);
    const uint32_t ie = wave_inclusive_scan(ve, lane);
    if (lane == 63) {
      wtot[0][wave] = ig;
      wtot[1][wave] = ie;
    }
    __syncthreads();
    uint32_t bg = 0, be = 0, tg = 0, te = 0;
    for (int w = 0; w < kTopkWaves; ++w) {
      const uint32_t xg = wtot[0][w], xe = wtot[1][w];
      if (w < wave) {
        bg += xg;
        be += xe;
      }
      tg += xg;
      te += xe;
    }
    if (c < a.n_chunks) {
      cnt[2 * c] = carry_gt + bg + ig - vg;
      cnt[2 * c + 1] = carry_eq + be + ie - ve;
    }
    carry_gt += tg;
    carry_eq += te;
    __syncthreads();   // hist and wtot are rewritten by the next group
  }
  if (tid == 0) {
    a.state[2 * h] = T;
    a.state[2 * h + 1] = need;
  }
}

// Compaction and gather, one workgroup per (chunk of kChunk keys, kv head).
// Thread t takes key i = c*kChunk + t.  Keys > T are all kept; of the keys == T
// the first `need` in index order are kept.  A kept key's output slot is the
// number of kept keys before it: (keys > T before it) + min(keys == T before it,
// need), from the chunk's counts plus wave ballots inside the chunk.  Kept keys
// are listed in LDS, then the workgroup copies their K and V head rows with
// 16-byte loads (consecutive threads on consecutive pieces of one row).
__global__ __launch_bounds__(kChunk) void topk_place_gather_kernel(const TopkArgs a) {
  __shared__ uint32_t wcnt[3][kChunk / 64];
  __shared__ int32_t kept_tok[kChunk], kept_pos[kChunk];
  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = a.L;
  const uint32_t l = (uint32_t)a.l;
  const int i = c * kChunk + tid;
  const bool valid = i < L;
  const uint32_t kk = valid ? order_key(a.scores[(size_t)h * L + i]) : 0u;
  const uint32_t T = a.state[2 * h];
  const uint32_t need = a.state[2 * h + 1];
  const uint32_t *cnt = a.chunk_counts + ((size_t)h * a.n_chunks + c) * 2;
  const bool gt = valid && kk > T;
  const bool eq = valid && kk == T;
  const unsigned long long bgt = __ballot(gt);
  const unsigned long long beq = __ballot(eq);
  if (lane == 0) {
    wcnt[0][wave] = (uint32_t)__popcll(bgt);
    wcnt[1][wave] = (uint32_t)__popcll(beq);
  }
  __syncthreads();
  uint32_t g = cnt[0] + lanes_below(bgt), e = cnt[1] + lanes_below(beq);
  for (int w = 0; w < wave; ++w) {
    g += wcnt[0][w];
    e += wcnt[1][w];
  }
  uint32_t pos = 0xffffffffu;
  if (gt) pos = g + min(e, need);
  else if (eq && e < need) pos = g + e;
  const bool keep = pos < l;
  const unsigned long long bk = __ballot(keep);
  if (lane == 0) wcnt[2][wave] = (uint32_t)__popcll(bk);
  __syncthreads();
  uint32_t slot = lanes_below(bk);
  uint32_t n_kept = 0;
  for (int w = 0; w < kChunk / 64; ++w) {
    if (w < wave) slot += wcnt[2][w];
    n_kept += wcnt[2][w];
  }
  if (keep) {
    a.idx[(size_t)h * l + pos] = i;
    kept_tok[slot] = i;
    kept_pos[slot] = (int32_t)pos;
  }
  __syncthreads();
  // copy: piece p of tensor t of kept entry e, for j = (e * 2 + t) * CH + p
  const int ch_log2 = (a.d == 128) ? 4 : 3;   // 16-byte pieces per head row: d / 8
  const int n_pieces = (int)n_kept << (ch_log2 + 1);
  const size_t row_stride = (size_t)a.Hkv * a.d;
  for (int j = tid; j < n_pieces; j += kChunk) {
    const int ent = j >> (ch_log2 + 1);
    const bool is_v = (j >> ch_log2) & 1;
    const int p = j & ((1 << ch_log2) - 1);
    const size_t src = (size_t)kept_tok[ent] * row_stride + (size_t)h * a.d + p * 8;
    const size_t dst = (size_t)kept_pos[ent] * row_stride + (size_t)h * a.d + p * 8;
    const uint4 x = *reinterpret_cast<const uint4 *>((is_v ? a.v : a.k) + src);
    *reinterpret_cast<uint4 *>((is_v ? a.vc : a.kc) + dst) = x;
  }
}

}  // namespace

// Workspace of the allocation-free entry point: one array per GPU, holding the
// top-l workspace of the last call made on that GPU.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device address);
// it uses the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) uint8_t scratch[kStaticTopkScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_topk_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t topk_workspace_bytes(int L, int Hkv) {
  const size_t n_chunks = ((size_t)L + kChunk - 1) / kChunk;
  const size_t bytes = (size_t)Hkv * 2 * sizeof(uint32_t) + (size_t)Hkv * n_chunks * 2 * sizeof(uint32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_topk_gather(TopkArgs &a, void *workspace, hipStream_t s) {
  a.n_chunks = (a.L + kChunk - 1) / kChunk;
  a.state = static_cast<uint32_t *>(workspace);
  a.chunk_counts = a.state + 2 * a.Hkv;
  if (a.L <= kLdsKeys) {
    hipLaunchKernelGGL((topk_select_kernel<true>), dim3(a.Hkv), dim3(kTopkThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((topk_select_kernel<false>), dim3(a.Hkv), dim3(kTopkThreads), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_place_gather_kernel, dim3(a.n_chunks, a.Hkv), dim3(kChunk), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
