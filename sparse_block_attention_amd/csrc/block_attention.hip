// APB per-host attention: local queries over [anchor | passing | local causal].
//
// Source: juejin.cn APB explainer, section "APB 的主要功能", bullet on
// computation (each host attends over anchor, passing and local blocks), and the
// arXiv abstract's "tailored FlashAttn kernel".  The mask reading (anchor and
// passing fully visible, local keys causal) follows from every anchor and
// passing token preceding every local token in the sequence.
//
// gfx950 design (one code path, instantiated for head_dim 64 and 128):
//  * Workgroup = NW wave64s; each wave owns 32*NSUB consecutive query rows of one
//    q head.  The grid walks (kv head, q tile longest-first, q head of the group)
//    and is remapped so that consecutive work items land on the same XCD: the q
//    heads sharing a kv head stream the same K/V tiles through one L2.
//  * K/V tiles of BN keys are staged through double-buffered LDS with register
//    prefetch of the next tile; one barrier per tile.  Segment tails and the
//    causal diagonal are masked; local tiles beyond a wave's last row are skipped.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the query row is the MFMA column,
//    so each lane holds the scores of one row (16 keys per 32-key block).  K rows
//    are stored in LDS in a permuted order chosen so that lane half h of the
//    accumulator holds keys 16h..16h+15 of the block, in order.  Those 16 values,
//    converted to bf16, are directly the B operand of O^T = V^T P^T: no
//    cross-lane movement of P.
//  * V is transposed into LDS (rows = head_dim) with a 16-byte XOR swizzle so
//    that both the transposing writes and the MFMA operand reads are free of
//    bank conflicts.
//  * Online softmax in the exp2 domain with the scale folded into one FMA; the
//    row max is exchanged between lane halves with v_permlane32_swap; the row
//    sum stays per lane until the end.  The running max is only moved when a
//    row's max grows by more than 2^8 (then O and the sum are rescaled); until
//    then probabilities are taken against the stale max, which is exact after
//    the final normalisation and keeps every p below 2^8.
#include "apb_internal.h"

#ifndef APB_ATTN_NSUB
#define APB_ATTN_NSUB 1
#endif
#ifndef APB_ATTN_BN
#define APB_ATTN_BN 64
#endif
#ifndef APB_ATTN_NW
#define APB_ATTN_NW 8
#endif
#ifndef APB_ATTN_WPE
#define APB_ATTN_WPE 2
#endif

namespace apb {
namespace {

constexpr float kLazyRescale = 8.0f;  // log2 units

__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS slot of key row `row` of a K tile: within each 32-row block, slot m holds
// key ((m%8)/4)*16 + (m/8)*4 + m%4, so MFMA output value i of lane half h is
// key 16h + i of the block.
__device__ __forceinline__ int k_slot(int row) {
  const int r = row & 31;
  return (row & ~31) + ((r & 15) >> 2) * 8 + (r >> 4) * 4 + (r & 3);
}

// 16-byte chunk swizzle of the transposed V tile (row = head-dim index).
__device__ __forceinline__ int v_swz(int d) { return (d ^ (d >> 3)) & 7; }

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) {
  return (lo16 & 0xffffu) | (hi16 << 16);
}

__device__ __forceinline__ uint32_t u16_at(const uint4 &x, int e) {
  const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

struct TileRef {
  const uint16_t *k, *v;
  int k0, seg_len, seg;  // seg: 0 anchor, 1 passing, 2 local
};

template <int D, int NSUB, int BN, int NW>
struct AttnCfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int BM = NW * 32 * NSUB;      // query rows per workgroup
  static constexpr int KP = D + 8;               // K row pitch in u16 (16 B pad)
  static constexpr int KS = BN * KP;             // K tile, u16
  static constexpr int VS = D * BN;              // transposed V tile, u16
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int KROWS = kThreads / CH;    // K rows loaded per pass
  static constexpr int KIT = BN / KROWS;         // K passes per thread
  static constexpr int KPT = BN * CH / kThreads; // V keys per thread
  static constexpr int NKB = BN / 32;            // 32-key blocks per tile
  static constexpr int DB = D / 32;              // 32-wide head-dim blocks of O
  static constexpr int KK = D / 16;              // MFMA k-steps over head_dim
  static constexpr int LDS_BYTES = 2 * (KS + VS) * 2;
  static_assert(KPT == 2 || KPT == 4 || KPT == 8, "V transpose expects 2, 4 or 8 keys per thread");
  static_assert(KIT >= 1 && KROWS * KIT == BN, "K tile split");
};

template <int D, int NSUB, int BN, int NW, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void block_attention_kernel(const AttnArgs a) {
  using C = AttnCfg<D, NSUB, BN, NW>;
  constexpr int BM = C::BM, KP = C::KP, KS = C::KS, VS = C::VS, CH = C::CH, KROWS = C::KROWS;
  constexpr int KIT = C::KIT, KPT = C::KPT, NKB = C::NKB, DB = C::DB, KK = C::KK;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KS + VS)];

  // ---- work item: XCD-aware remap, then (kv head, q tile longest-first, member)
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int w = (bid % kNumXcd) * (nb / kNumXcd) + bid / kNumXcd;
  if (w >= a.n_work) return;
  const int per_h = a.n_qtiles * a.g;
  const int h = w / per_h;
  const int rem = w - h * per_h;
  const int qtile = a.n_qtiles - 1 - rem / a.g;
  const int qhead = a.qhead_of_slot[h * a.g + rem % a.g];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int r0 = qtile * BM;
  const int rw = r0 + wave * 32 * NSUB;   // first row of this wave
  const size_t q_stride = (size_t)a.Hq * D;
  const size_t kv_stride = (size_t)a.Hkv * D;

  // ---- Q fragments (B operand of S^T = K Q^T): row lrow, head-dim 16kk + 8half..+7
  bf16x8 qf[NSUB][KK];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int row = rw + s * 32 + lrow;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (row < a.L) {
        qf[s][kk] = *reinterpret_cast<const bf16x8 *>(a.q + row * q_stride + qhead * D + kk * 16 + half * 8);
      } else {
        qf[s][kk] = bf16x8{};
      }
    }
  }

  // ---- tile list: anchor tiles, passing tiles, local tiles up to the last row
  const int nA = (a.A + BN - 1) / BN;
  const int nP = (a.P + BN - 1) / BN;
  const int last_row = min(r0 + BM, a.L);
  const int nL = (last_row + BN - 1) / BN;
  const int n_tiles = nA + nP + nL;

  auto tile_ref = [&](int t) {
    TileRef r;
    if (t < nA) {
      r.k = a.ka; r.v = a.va; r.k0 = t * BN; r.seg_len = a.A; r.seg = 0;
    } else if (t < nA + nP) {
      r.k = a.kp; r.v = a.vp; r.k0 = (t - nA) * BN; r.seg_len = a.P; r.seg = 1;
    } else {
      r.k = a.kl; r.v = a.vl; r.k0 = (t - nA - nP) * BN; r.seg_len = a.L; r.seg = 2;
    }
    return r;
  };

  uint4 kreg[KIT];
  uint4 vreg[KPT];
  const int chunk = tid % CH;
  const int kg = tid / CH;

  auto load_regs = [&](const TileRef &t) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int key = t.k0 + it * KROWS + kg;
      if (key < t.seg_len) {
        kreg[it] = *reinterpret_cast<const uint4 *>(t.k + key * kv_stride + h * D + chunk * 8);
      } else {
        kreg[it] = uint4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int key = t.k0 + kg * KPT + j;
      if (key < t.seg_len) {
        vreg[j] = *reinterpret_cast<const uint4 *>(t.v + key * kv_stride + h * D + chunk * 8);
      } else {
        vreg[j] = uint4{0, 0, 0, 0};
      }
    }
  };

  auto store_lds = [&](uint16_t *buf) {
    uint16_t *Ks = buf;
    uint16_t *Vt = buf + KS;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int row = it * KROWS + kg;
      *reinterpret_cast<uint4 *>(Ks + k_slot(row) * KP + chunk * 8) = kreg[it];
    }
    const int key0 = kg * KPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = chunk * 8 + e;
      uint16_t *dst = Vt + d * BN + (((key0 >> 3) ^ v_swz(d)) << 3) + (key0 & 7);
      if constexpr (KPT == 8) {
        uint4 p;
        p.x = pack2(u16_at(vreg[0], e), u16_at(vreg[1], e));
        p.y = pack2(u16_at(vreg[2], e), u16_at(vreg[3], e));
        p.z = pack2(u16_at(vreg[4], e), u16_at(vreg[5], e));
        p.w = pack2(u16_at(vreg[6], e), u16_at(vreg[7], e));
        *reinterpret_cast<uint4 *>(dst) = p;
      } else if constexpr (KPT == 4) {
        uint2 p;
        p.x = pack2(u16_at(vreg[0], e), u16_at(vreg[1], e));
        p.y = pack2(u16_at(vreg[2], e), u16_at(vreg[3], e));
        *reinterpret_cast<uint2 *>(dst) = p;
      } else {
        *reinterpret_cast<uint32_t *>(dst) = pack2(u16_at(vreg[0], e), u16_at(vreg[1], e));
      }
    }
  };

  // ---- accumulators
  f32x16 acc[NSUB][DB];
  float m_run[NSUB], l_run[NSUB];
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    m_run[s] = -INFINITY;
    l_run[s] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[s][db] = f32x16{};
  }
  const float sl2 = a.scale_log2;

  // ---- prologue
  {
    TileRef t0 = tile_ref(0);
    load_regs(t0);
    store_lds(smem);
    __syncthreads();
  }

  for (int t = 0; t < n_tiles; ++t) {
    const TileRef cur = tile_ref(t);
    if (t + 1 < n_tiles) load_regs(tile_ref(t + 1));

    const uint16_t *Ks = smem + (t & 1) * (KS + VS);
    const uint16_t *Vt = Ks + KS;
    const bool wave_active = !(cur.seg == 2 && cur.k0 > rw + 32 * NSUB - 1);
    if (wave_active) {
      // S^T = K Q^T, one 32-key block at a time
      f32x16 sacc[NSUB][NKB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sacc[s][kb] = f32x16{};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (kb * 32 + lrow) * KP + kk * 16 + half * 8);
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            sacc[s][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s][kk], sacc[s][kb], 0, 0, 0);
        }
      }

      const bool need_mask = (cur.k0 + BN > cur.seg_len) || (cur.seg == 2 && cur.k0 + BN - 1 > rw);
      bf16x8 pf[NSUB][NKB][2];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (need_mask) {
          const int row = rw + s * 32 + lrow;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = cur.k0 + kb * 32 + half * 16 + i;
              const bool dead = key >= cur.seg_len || (cur.seg == 2 && key > row);
              if (dead) sacc[s][kb][i] = -INFINITY;
            }
          }
        }
        float mx = sacc[s][0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[s][kb][i]);
        mx = half_swap_max(mx);
        const float m_cand = fmaxf(m_run[s], mx * sl2);
        const bool grow = m_cand > m_run[s] + kLazyRescale;
        if (__ballot(grow)) {
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[s] - m_cand) : 1.f;
          m_run[s] = grow ? m_cand : m_run[s];
          l_run[s] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[s][db] *= alpha;
        }
        const float m_use = (m_run[s] == -INFINITY) ? 0.f : m_run[s];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            uint32_t w4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s][kb][c * 8 + 2 * j], sl2, -m_use));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s][kb][c * 8 + 2 * j + 1], sl2, -m_use));
              psum += p0 + p1;
              w4[j] = bf16x2_bits(p0, p1);
            }
            pf[s][kb][c] = __builtin_bit_cast(bf16x8, (uint4{w4[0], w4[1], w4[2], w4[3]}));
          }
        }
        l_run[s] += psum;
      }

      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int lchunk = kb * 4 + half * 2 + c;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + lrow;
            const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(Vt + d * BN + ((lchunk ^ v_swz(d)) << 3));
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
              acc[s][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[s][kb][c], acc[s][db], 0, 0, 0);
          }
        }
      }
    }

    if (t + 1 < n_tiles) store_lds(smem + ((t + 1) & 1) * (KS + VS));
    __syncthreads();
  }

  // ---- epilogue: normalise, write O (bf16) and LSE (natural log)
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int row = rw + s * 32 + lrow;
    const float l_tot = half_swap_sum(l_run[s]);
    const float inv = 1.f / l_tot;
    if (row < a.L) {
      uint16_t *orow = a.out + row * q_stride + qhead * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          uint2 p;
          p.x = bf16x2_bits(acc[s][db][g4 * 4 + 0] * inv, acc[s][db][g4 * 4 + 1] * inv);
          p.y = bf16x2_bits(acc[s][db][g4 * 4 + 2] * inv, acc[s][db][g4 * 4 + 3] * inv);
          *reinterpret_cast<uint2 *>(orow + db * 32 + g4 * 8 + half * 4) = p;
        }
      }
      if (a.lse != nullptr && half == 0) {
        a.lse[(size_t)qhead * a.L + row] = (m_run[s] + __log2f(l_tot)) * 0.69314718055994531f;
      }
    }
  }
}

template <int D, int NSUB, int BN, int NW, int WPE>
hipError_t launch_impl(AttnArgs &a, hipStream_t s) {
  using C = AttnCfg<D, NSUB, BN, NW>;
  a.n_qtiles = (a.L + C::BM - 1) / C::BM;
  a.n_work = a.n_qtiles * a.Hq;
  const int grid = (a.n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL((block_attention_kernel<D, NSUB, BN, NW, WPE>), dim3(grid), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_attention(AttnArgs &a, int head_dim, hipStream_t s) {
  if (head_dim == 128) return launch_impl<128, APB_ATTN_NSUB, APB_ATTN_BN, APB_ATTN_NW, APB_ATTN_WPE>(a, s);
  return launch_impl<64, 1, 64, 4, 2>(a, s);
}

}  // namespace apb
