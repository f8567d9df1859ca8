// APB per-host attention: local queries over [anchor | passing | local causal].
//
// Source: juejin.cn APB explainer, section "APB 的主要功能", bullet on
// computation (each host attends over anchor, passing and local blocks), and the
// arXiv abstract, which names a FlashAttention kernel adapted to APB.  The mask
// reading (anchor and passing fully visible, local keys causal) follows from
// every anchor and passing token preceding every local token in the sequence.
//
// gfx950 design (one code path, instantiated for head_dim 64 and 128, and for
// 128 also with 4-wave workgroups for problems with few work items):
//  * Workgroup = NW wave64s; each wave owns 32*NSUB consecutive query rows of one
//    q head.  The grid walks (kv head, q tile longest-first, q head of the group)
//    and is remapped so that consecutive work items land on the same XCD: the q
//    heads sharing a kv head stream the same K/V tiles through one L2.
//  * K/V tiles of BN keys go HBM -> LDS by LDS-DMA (buffer_load_dwordx4 ... lds):
//    no staging registers, no LDS store instructions, and per-lane source offsets
//    fixed for the whole kernel.  A per-tile buffer descriptor ends at the
//    segment's last row, so rows past it read as zeros.  Two LDS buffers: tile
//    t+1 is in flight while tile t is consumed (the DMA has one tile of compute
//    to land); one barrier per tile.  Segment tails and
//    the causal diagonal are masked; local tiles past a wave's rows are skipped.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the query row is the MFMA column,
//    so each lane holds the scores of one row (16 keys per 32-key block).  K rows
//    sit in LDS in a permuted slot order chosen so that lane half h of the
//    accumulator holds keys 16h..16h+15 of the block, in order; those values,
//    converted to bf16, are directly the B operand of O^T = V^T P^T (no lane
//    movement of P).  K rows are padded to an odd number of 16-byte chunks, so
//    the reads are conflict-free with the head-dim offset as an immediate.
//  * V stays row-major in LDS (32-byte granules XOR-swizzled by key) and the A
//    operand of O^T = V^T P^T is read with ds_read_b64_tr_b16, which transposes
//    4 keys x 16 head-dim values across each 16-lane group.
//  * Online softmax in the exp2 domain with the scale folded into one FMA.  The
//    common path has no row max: probabilities are taken against the running
//    reference, and only a wave in which some lane's tile sum exceeds 2^32 (or is
//    not finite, as on the first tile) computes the true max, rescales O and the
//    sum, and recomputes.  The final normalisation makes this exact; every p
//    stays far below the fp32 and bf16 range.  The row max is exchanged between
//    lane halves with v_permlane32_swap; row sums stay per lane until the end.
//  * The tile loop runs two tiles per iteration, so both buffers' LDS addresses
//    are loop-invariant registers plus immediates, and walks the tiles with a
//    cursor (pointer bumps; a branch only where a segment ends).  Each tile
//    issues its K reads before it sets up the next tile's DMA, and reads its
//    first V fragments before the softmax.
#include "apb_internal.h"

// Workgroup shape and tile size of the head_dim 128 instance (the defaults are
// the measured best; the head_dim 64 instance, and the head_dim 128 one used for
// problems with few work items, are fixed at 1, 64, 4, 2).
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
#ifndef APB_ATTN_SCHED
#define APB_ATTN_SCHED 1
#endif

namespace apb {
namespace {

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

__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

// One K/V tile: its segment (0 anchor, 1 passing, 2 local), its first key k0
// within the segment, the segment length, and K/V pointers at row k0.
struct TileRef {
  const uint16_t *k, *v;
  int k0, seg_len, seg;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Inverse of k_slot: key row stored in LDS slot `slot` of a K tile.
__device__ __forceinline__ int slot_key(int slot) {
  const int u = slot & 31;
  return (slot & ~31) + ((u & 7) >> 2) * 16 + (u >> 3) * 4 + (u & 3);
}

template <int D, int NSUB, int BN, int NW>
struct AttnCfg {
  static constexpr int kThreads = 64 * NW;
  static constexpr int BM = NW * 32 * NSUB;      // query rows per workgroup
  static constexpr int ROWB = D * 2;             // bytes per V row in LDS (no padding)
  static constexpr int TILE_BYTES = BN * ROWB;   // one V tile
  static constexpr int KROWB = ROWB + 16;        // bytes per K row in LDS: one 16-byte pad
  static constexpr int KTB = BN * KROWB;         // one K tile
  static constexpr int SB = KTB + TILE_BYTES;    // one LDS buffer: K tile, then V tile
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int GR = D / 16;              // 32-byte granules per row
  static constexpr int KI = TILE_BYTES / 1024 / NW;  // 1 KB LDS-DMA loads of V per wave per tile
  static constexpr int NKL = KTB / 1024;             // 1 KB LDS-DMA loads of one K tile
  static constexpr int KIK = (NKL + NW - 1) / NW;    // K loads per wave (the last ones: low waves only)
  static constexpr int NKB = BN / 32;            // 32-key blocks per tile
  static constexpr int DB = D / 32;              // 32-wide head-dim blocks of O
  static constexpr int KK = D / 16;              // MFMA k-steps over head_dim
  static_assert(KI >= 1 && KI * 1024 * NW == TILE_BYTES, "tile split over LDS-DMA loads");
  static_assert(NKL * 1024 == KTB && SB % 1024 == 0, "padded K tile split over LDS-DMA loads");
};

// V tile granule swizzle: 32-byte granule g of key row `key` sits at g ^ vsw(key).
template <int GR>
__device__ __forceinline__ int vsw(int key) { return (2 * (key & 3)) & (GR - 1); }

// Issue this wave's LDS-DMA loads of one K tile (loads wave, wave + NW, ... of the
// NKL 1 KB pieces) and one V tile (KI x 1 KB).  The buffer descriptors cover rows
// [k0, seg_len) of the segment (at most BN), so rows past a segment's end read as
// zeros.  (The body exists only in the device pass: the host pass has no
// buffer-descriptor type.)
template <int KI, int KIK, int NKL, int NW, int BN>
__device__ __forceinline__ void issue_tile_loads(const TileRef &t, int kv_row_bytes, int wave, uint8_t *kdst,
                                                 uint8_t *vdst, const int (&koff)[KIK], const int (&voff)[KI]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int valid_bytes = min(t.seg_len - t.k0, BN) * kv_row_bytes;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void *)t.k, 0, valid_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void *)t.v, 0, valid_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < KIK; ++i) {
    if (i * NW + NW <= NKL || i * NW + wave < NKL)  // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(kdst + i * NW * 1024), 16, koff[i], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < KI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vdst + i * 1024), 16, voff[i], 0, 0, 0);
#endif
}

constexpr float kRescaleSum = 4294967296.0f;  // 2^32: a tile sum above this moves the max

template <int D, int NSUB, int BN, int NW, int WPE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(WPE, 8)))
void block_attention_kernel(const AttnArgs a) {
  using C = AttnCfg<D, NSUB, BN, NW>;
  constexpr int BM = C::BM, ROWB = C::ROWB, TB = C::TILE_BYTES, CH = C::CH, GR = C::GR, KI = C::KI;
  constexpr int KROWB = C::KROWB, KTB = C::KTB, SB = C::SB, KIK = C::KIK, NKL = C::NKL;
  constexpr int NKB = C::NKB, DB = C::DB, KK = C::KK;

  // [buffer][K tile | V tile]; tile t uses buffer t % 2 and tile t + 1 is in
  // flight while tile t is consumed.
  constexpr int NBUF = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * SB];

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS targets stay scalar
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int r0 = qtile * BM;
  const int rw = r0 + wave * 32 * NSUB;   // first row of this wave
  const size_t q_stride = (size_t)a.Hq * D;
  const int kv_row_bytes = a.Hkv * D * 2;

  // ---- zero both LDS buffers once: rows past a segment end never hold NaN
  for (int i = tid; i < NBUF * SB / 16; i += C::kThreads) reinterpret_cast<uint4 *>(smem)[i] = uint4{0, 0, 0, 0};

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

  // ---- per-lane source offsets of the LDS-DMA loads (fixed for the whole kernel).
  // Lane p of a load writes 16 bytes at p*16 of the load's 1 KB.  K load i of this
  // wave fills bytes [(i*NW + wave) * 1024, +1024) of the padded K tile: LDS row
  // `row` (KROWB bytes) is slot `row`, holding key slot_key(row), chunks in order,
  // then a pad (filled with a copy of the last chunk).  V load i fills bytes
  // [(wave*KI + i) * 1024, +1024) of the V tile.
  int koff[KIK], voff[KI];
#pragma unroll
  for (int i = 0; i < KIK; ++i) {
    const int pos = (i * NW + wave) * 64 + lane;  // 16-byte position in the padded K tile
    const int row = min(pos / (CH + 1), BN - 1);   // (rows past BN: a load that is never issued)
    const int pc = min(pos % (CH + 1), CH - 1);
    koff[i] = slot_key(row) * kv_row_bytes + h * D * 2 + pc * 16;
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int pos = (wave * KI + i) * 64 + lane;  // 16-byte position in the V tile
    const int row = pos / CH;
    const int pc = pos % CH;
    // V: LDS row = key; granule pc/2 holds granule (pc/2) ^ vsw(key).
    const int gi = (pc >> 1) ^ vsw<GR>(row);
    voff[i] = row * kv_row_bytes + h * D * 2 + (gi * 2 + (pc & 1)) * 16;
  }

  // ---- tile list: anchor tiles, passing tiles, local tiles up to the last row
  const int nA = (a.A + BN - 1) / BN;
  const int nP = (a.P + BN - 1) / BN;
  const int last_row = min(r0 + BM, a.L);
  const int nL = a.use_local ? (last_row + BN - 1) / BN : 0;
  const int n_tiles = nA + nP + nL;

  // Tiles are walked by a cursor: the next tile is the current one advanced by BN
  // rows, or the first tile of the next non-empty segment.  The segment pointers
  // and lengths are read from the arguments here, before the loop, and the empty
  // asm makes them live in registers from this point: a kernel-argument load left
  // for the rare segment switch would be outstanding at the loop's first LDS waits.
  const uint16_t *kp = a.kp, *vp = a.vp, *kl = a.kl, *vl = a.vl;
  asm volatile("" : "+s"(kp), "+s"(vp), "+s"(kl), "+s"(vl));
  const int seg_P = a.P, seg_L = a.L;
  const int tile_elems = BN * (kv_row_bytes / 2);
  TileRef first;
  if (a.A > 0) first = TileRef{a.ka, a.va, 0, a.A, 0};
  else if (seg_P > 0) first = TileRef{kp, vp, 0, seg_P, 1};
  else first = TileRef{kl, vl, 0, seg_L, 2};
  auto advance = [&](const TileRef &c) {
    TileRef n{c.k + tile_elems, c.v + tile_elems, c.k0 + BN, c.seg_len, c.seg};
    if (c.seg < 2 && n.k0 >= c.seg_len) {  // wave-uniform, once per segment
      if (c.seg == 0 && seg_P > 0) n = TileRef{kp, vp, 0, seg_P, 1};
      else n = TileRef{kl, vl, 0, seg_L, 2};
    }
    return n;
  };

  // ---- per-lane LDS read offsets
  // K (A operand of S^T): slot kb*32 + lrow, chunk 2kk + half.  The padded row
  // stride is an odd number of 16-byte chunks, so 16 consecutive slots start on 16
  // distinct 16-byte bank groups (64 banks x 4 bytes) and the reads are
  // conflict-free; kb and kk then enter the address as immediate offsets.
  const int k_rd = lrow * KROWB + half * 16;
  // V (A operand of O^T via the transposing read): 16-lane group gq reads keys
  // base + (lane%16)/4 at head-dim db*32 + (gq%2)*16 + 4*(lane%4) .. +3.
  const int gq = lane >> 4;
  const int v_key = half * 16 + ((lane & 15) >> 2);
  const int v_fx = vsw<GR>(v_key);
  int v_rd[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_rd[db] = v_key * ROWB + (((db * 2 + (gq & 1)) ^ v_fx) * 32) + (lane & 3) * 8;

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
  // The softmax scale is first used inside the tile loop.  The empty asm reads
  // it here, so its scalar load has landed before the loop.  Otherwise the load
  // would be outstanding at the loop's first waits, and since scalar loads can
  // return out of order, every wait for an LDS read in the loop would have to be
  // a full lgkmcnt(0) instead of waiting for just the reads it needs.
  float sl2 = a.scale_log2;
  asm volatile("" : "+s"(sl2));

  // ---- prologue
  // LDS zeroed in every wave before the first DMA lands.  No wait for the q loads
  // here: they stay in flight beside the first tile's DMA.
  barrier_lds_drained();
  if (n_tiles > 0)
    issue_tile_loads<KI, KIK, NKL, NW, BN>(first, kv_row_bytes, wave, smem + wave * 1024,
                                           smem + KTB + wave * KI * 1024, koff, voff);
  wait_vmcnt<0>();
  __syncthreads();

  // One tile: prefetch tile `nx` into `nxt`, consume tile `cur` from `cur_buf`.  The two
  // buffers are distinct; saying so (__restrict__) lets the compiler skip the
  // wait for the in-flight DMA before reading `cur`.
  auto tile_step = [&](const TileRef &cur, const TileRef &nx, const uint8_t *__restrict__ cur_buf,
                       uint8_t *__restrict__ nxt, bool prefetch) {
    const uint8_t *Ks = cur_buf;
    const uint8_t *Vs = cur_buf + KTB;
    const bool wave_active = !(cur.seg == 2 && cur.k0 > rw + 32 * NSUB - 1);
    // K fragments of block kb+1 are read into the slots that block kb has used,
    // so KK reads are in flight ahead of the MFMAs.  The first reads go out
    // before the next tile's DMA is set up, so their latency covers that work.
    const uint8_t *kr = Ks + k_rd;
    bf16x8 kf[KK];
    if (wave_active) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + kk * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (prefetch) {
      issue_tile_loads<KI, KIK, NKL, NW, BN>(nx, kv_row_bytes, wave, nxt + wave * 1024,
                                             nxt + KTB + wave * KI * 1024, koff, voff);
    }
    __builtin_amdgcn_sched_barrier(0);
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
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            sacc[s][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[s][kk], sacc[s][kb], 0, 0, 0);
          if (kb + 1 < NKB) kf[kk] = *reinterpret_cast<const bf16x8 *>(kr + (kb + 1) * 32 * KROWB + kk * 32);
        }
      }
#if APB_ATTN_SCHED
      // K reads run KK MFMAs ahead of their use
#pragma unroll
      for (int i = 0; i < (NKB - 1) * KK * NSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i % NSUB == NSUB - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KK * NSUB, 0);
#endif

      // V fragment (A operand of O^T += V^T P^T) for keys kb*32 + c*8 .. +7 and
      // head-dim block db: 8 keys x 32 head-dim rows from two transposing reads.
      auto v_frag = [&](int kb, int c, int db) {
        const uint8_t *vb = Vs + (kb * 32 + c * 8) * ROWB + v_rd[db];
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(vb));
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(vb + 4 * ROWB));
        return __builtin_bit_cast(bf16x8, (__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
      };
      // The first DB fragments are read before the softmax, which hides their latency.
      bf16x8 vfr[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) vfr[db] = v_frag(0, 0, db);

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
        // Probabilities against the running reference m_run; a wave whose tile sum
        // is too large (or not finite, as on the first tile) moves the reference to
        // the true max, rescales O and the sum, and recomputes.
        auto exp_tile = [&](float m_use) {
          float psum;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              uint32_t w4[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[s][kb][c * 8 + 2 * j], sl2, -m_use));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[s][kb][c * 8 + 2 * j + 1], sl2, -m_use));
                psum = (kb == 0 && c == 0 && j == 0) ? p0 + p1 : psum + (p0 + p1);
                w4[j] = bf16x2_bits(p0, p1);
              }
              pf[s][kb][c] = __builtin_bit_cast(bf16x8, (uint4{w4[0], w4[1], w4[2], w4[3]}));
            }
          }
          return psum;
        };
        float psum = exp_tile(m_run[s]);
        if (__ballot(!(psum <= kRescaleSum))) {
          float mx = sacc[s][0][0];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[s][kb][i]);
          mx = half_swap_max(mx);
          const float m_new = fmaxf(m_run[s], mx * sl2);
          const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_use);
          m_run[s] = m_new;
          l_run[s] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[s][db] *= alpha;
          psum = exp_tile(m_use);
        }
        l_run[s] += psum;
      }

      // O^T += V^T P^T; the next (kb, c) fragment of head-dim block db is read into
      // the slot its MFMA has just used
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
          for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
              acc[s][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[db], pf[s][kb][c], acc[s][db], 0, 0, 0);
            if (kb * 2 + c + 1 < NKB * 2) vfr[db] = v_frag(c == 1 ? kb + 1 : kb, c ^ 1, db);
          }
        }
      }
#if APB_ATTN_SCHED
      // transposing V reads run DB MFMAs ahead of their use
#pragma unroll
      for (int i = 0; i < NKB * 2 * DB - DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NSUB, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, DB * NSUB, 1);
#endif
    }
  };

  // Tile t+1 must have landed in every wave before the barrier that ends tile t.
  auto tile_end = [&]() {
    wait_vmcnt<0>();
    barrier_lds_drained();
  };
  // Two tiles per iteration, so that each one's buffers are constants and the LDS
  // read addresses need no per-tile add.
  TileRef cur = first;
  int t = 0;
  for (; t + 1 < n_tiles; t += 2) {
    TileRef nx = advance(cur);
    tile_step(cur, nx, smem, smem + SB, true);
    tile_end();
    cur = nx;
    nx = advance(cur);
    tile_step(cur, nx, smem + SB, smem, t + 2 < n_tiles);
    tile_end();
    cur = nx;
  }
  if (t < n_tiles) {
    tile_step(cur, cur, smem, smem + SB, false);
    tile_end();
  }

  // ---- epilogue: normalise, write O (bf16) and LSE (natural log)
#pragma unroll
  for (int s = 0; s < NSUB; ++s) {
    const int row = rw + s * 32 + lrow;
    const float l_tot = half_swap_sum(l_run[s]);
    // l_tot == 0 only when the row saw no key at all (segments left out): O = 0, lse = -inf
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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
        a.lse[(size_t)qhead * a.L + row] =
            l_tot > 0.f ? (m_run[s] + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
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

// Work items of 256 query rows below which the head_dim 128 attention uses
// 128-row workgroups (4 waves, two workgroups per CU): with fewer than four
// 256-row items per CU the causal imbalance between q tiles leaves CUs idle, and
// twice as many smaller items balance better.  Measured: the anchor's own causal
// attention (A = 2048, 32 q heads: 256 items) 59.9 -> 54.0 us, at A = 4096 with
// 40 heads 199 -> 182 us; with 2048 items (a Llama-3.1-8B host block, or the
// anchor at A = 16384) the 256-row workgroups are 5-6% faster.
constexpr long long kSmallAttnItems = 1024;

hipError_t launch_block_attention(AttnArgs &a, int head_dim, hipStream_t s) {
  if (head_dim == 128) {
    const long long items256 = (long long)((a.L + 255) / 256) * a.Hq;
    if (items256 < kSmallAttnItems) return launch_impl<128, 1, 64, 4, 2>(a, s);
    return launch_impl<128, APB_ATTN_NSUB, APB_ATTN_BN, APB_ATTN_NW, APB_ATTN_WPE>(a, s);
  }
  return launch_impl<64, 1, 64, 4, 2>(a, s);
}

}  // namespace apb
