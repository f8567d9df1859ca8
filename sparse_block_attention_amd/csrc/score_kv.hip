// APB step 1: per-kv-head importance score of each local token.
//
// Stand-in for Locret's retaining heads (juejin.cn APB explainer, section
// "APB 的主要功能": each host compresses its KV cache with retaining heads;
// section "APB 的技术原理": the query sits at the start of the anchor so the
// compressor sees it).  For kv head h and token t:
//   x = [q[t, G_h[0]]; ...; q[t, G_h[g-1]]; k[t, h]; v[t, h]]
//   s = w2[h] . relu(W1[h] x + b1[h]) + b2[h]
//
// gfx950 design: a workgroup takes 128*TH tokens of one kv head and all Hs
// hidden units: Z^T = W1 X^T on v_mfma_f32_32x32x16_bf16 (M = hidden, N =
// tokens, K = (g+2)d), K walked in 64-wide chunks.  4*TH waves: wave w owns
// hidden quarter w%4 (blocks w%4, w%4 + 4, ...) for token half w/4 (128 tokens),
// so a W1 element is read from LDS by TH waves.  X and W1 chunks reach LDS by
// LDS-DMA (buffer_load ... lds) through a 2-deep ring: the next chunk is in
// flight while one is consumed.  A chunk row is 128 bytes, one whole cache line
// of the token's (or W1 row's) data: with 64-byte rows (32-wide chunks) each
// 1 KB load touched 16 half-used lines and kept the texture unit twice as busy
// per byte (64-wide chunks: 5-7% faster, texture busy cycles -31%).  Every
// workgroup streams its head's whole W1 from L2, so TH = 2 (256 tokens, one
// workgroup per CU) halves that L2 traffic against TH = 1 (128 tokens, two
// workgroups per CU).  The 16-byte pieces of a row are XOR-swizzled by row so
// the MFMA operand reads are free of bank conflicts.  The epilogue adds b1,
// applies ReLU and the w2 dot product in fp32, and sums the four hidden
// quarters' partial dot products through LDS.  Work items are grouped by kv
// head onto XCDs so a head's W1 stays in one L2.
#include <stddef.h>

#include "lds_dma.h"

namespace apb {
namespace {

#ifndef APB_SCORE_TH
#define APB_SCORE_TH 2
#endif
constexpr int kTH = APB_SCORE_TH;  // token halves (of 128 tokens) per workgroup
constexpr int kKC = 64;            // K chunk (elements of x)
#ifndef APB_SCORE_RING
#define APB_SCORE_RING 2
#endif
constexpr int kRing = APB_SCORE_RING;  // LDS ring depth (chunks in flight: kRing - 1)
constexpr int kRowB = kKC * 2;     // bytes per chunk row (128: whole cache lines)
constexpr int kXL = 4;             // X loads per wave per chunk (32 rows x 128 bytes)

// Piece swizzle of 128-byte chunk rows: 16-byte piece p of row r sits at p ^ swz(r),
// so 16 consecutive rows reading the same piece hit 16 distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int TH>
struct ScoreCfg {
  static constexpr int kWaves = 4 * TH;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTok = 128 * TH;          // tokens per workgroup
  static constexpr int kXB = kTok * kRowB;       // X chunk bytes
};

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS-DMA loads one wave issues per chunk: kXL of X plus W1 loads wave, wave+NW, ...
template <int WI_TOTAL, int NW>
__device__ __forceinline__ int loads_per_chunk(int wave) {
  return kXL + (WI_TOTAL > wave ? (WI_TOTAL - wave + NW - 1) / NW : 0);
}

// Where chunk c comes from.
struct ChunkSrc {
  const uint16_t *x;  // first element of the chunk in token row t0 of its tensor
  int x_valid;        // bytes of valid rows from x (range of the descriptor)
  const int *xo;      // this lane's offsets for its kXL X loads
  const uint16_t *w;  // W1 column offset of the chunk
};

// Per-workgroup constants needed to locate a chunk's sources.
struct SrcCtx {
  const uint16_t *q0, *k0, *v0;  // token row t0 of q, k, v
  const uint16_t *w1h;           // W1 of this kv head
  int xq_valid, xkv_valid;       // descriptor ranges for q rows and k/v rows
  const int *xq, *xkv;           // lane offsets of the kXL X loads, q and k/v strides
  int g, d;
};

// LDS reads in the main loop go through __restrict__ parameters (here and in
// score_chunk): the alias scopes that gives them tell the compiler that the
// LDS-DMA loads in flight write elsewhere, so it adds no wait for those loads
// before the reads.  The DMA itself is issued outside any such function, so it
// carries no alias metadata of its own.
__device__ __forceinline__ int lds_read_int(const int *__restrict__ tab, int i) { return tab[i]; }

// Sources of chunk c: segment seg = c*32/d of x, element offset from seg_off.
__device__ __forceinline__ ChunkSrc chunk_src(const SrcCtx &cx, const int *seg_off, int c) {
  ChunkSrc s;
  const int p0 = c * kKC;
  const int seg = p0 / cx.d;
  const int e0 = p0 - seg * cx.d;
  const int so = __builtin_amdgcn_readfirstlane(lds_read_int(seg_off, seg)) + e0;
  if (seg < cx.g) {
    s.x = cx.q0 + so;
    s.x_valid = cx.xq_valid;
    s.xo = cx.xq;
  } else {
    s.x = (seg == cx.g ? cx.k0 : cx.v0) + so;
    s.x_valid = cx.xkv_valid;
    s.xo = cx.xkv;
  }
  s.w = cx.w1h + p0;
  return s;
}

// Issue this wave's LDS-DMA loads of one chunk into ring slot `slot`: X rows
// wave*32 .. wave*32+31, and W1 loads wave, wave+NW, ...
template <int WI_TOTAL, int NW, int XB>
__device__ __forceinline__ void issue_chunk(const ChunkSrc &s, uint8_t *slot, int w_valid, int wo_base,
                                            int w_rowstep, int wave) {
  uint8_t *xd = slot + wave * kXL * 1024;
#pragma unroll
  for (int i = 0; i < kXL; ++i) dma_1k(s.x, s.x_valid, s.xo[i], xd + i * 1024);
#pragma unroll
  for (int j = 0; j < (WI_TOTAL + NW - 1) / NW; ++j) {
    const int li = wave + NW * j;  // W1 load index: rows li*8 .. li*8+7
    if (li < WI_TOTAL) dma_1k(s.w, w_valid, wo_base + li * 8 * w_rowstep, slot + XB + li * 1024);
  }
}

// Accumulate K chunk `cur` into acc: Z^T[hidden block, token block] += W1 X^T,
// for hidden quarter hq and token half th.
template <int HB, int XB>
__device__ __forceinline__ void score_chunk(f32x16 (&acc)[(HB + 3) / 4][4], const uint8_t *__restrict__ cur,
                                            int hq, int th, int lrow, int half) {
  constexpr int MBW = (HB + 3) / 4;
  const uint8_t *ws = cur + XB;
#pragma unroll
  for (int kk = 0; kk < kKC / 16; ++kk) {
    const int lp = 2 * kk + half;
    bf16x8 xf[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int r = (th * 4 + tb) * 32 + lrow;
      xf[tb] = *reinterpret_cast<const bf16x8 *>(cur + r * kRowB + ((lp ^ swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int mb = hq + 4 * j;
      if (mb < HB) {
        const int r = mb * 32 + lrow;
        const bf16x8 wf = *reinterpret_cast<const bf16x8 *>(ws + r * kRowB + ((lp ^ swz(r)) * 16));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          acc[j][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[tb], acc[j][tb], 0, 0, 0);
      }
    }
  }
}

template <int HB, int TH>  // hidden in (32 * HB - 32, 32 * HB]; 128 * TH tokens per workgroup
__global__ __launch_bounds__(ScoreCfg<TH>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void score_kv_kernel(const ScoreArgs a) {
  using C = ScoreCfg<TH>;
  constexpr int kThreads = C::kThreads, kTok = C::kTok, kXB = C::kXB, NW = C::kWaves;
  constexpr int HS = 32 * HB;
  constexpr int MBW = (HB + 3) / 4;          // hidden blocks per wave (blocks hq, hq+4, ...)
  constexpr int WB = HS * kRowB;             // W1 chunk bytes
  constexpr int WI_TOTAL = WB / 1024;        // 1 KB loads per W1 chunk
  constexpr int SLOT = kXB + WB;
  static_assert(WB % 1024 == 0, "W1 chunk split");
  static_assert(NW % 2 == 0, "W1 load index parity follows the wave's");

  // One LDS object, carved by hand.  With several, the compiler tags each LDS-DMA
  // load with its object's alias scope and then, unable to tell ring slots
  // apart, waits for every such load before each LDS read of the ring.
  constexpr int kOffB1 = kRing * SLOT;
  constexpr int kOffW2 = kOffB1 + HS * 4;
  constexpr int kOffRed = kOffW2 + HS * 4;
  constexpr int kOffSeg = kOffRed + 4 * kTok * 4;
  constexpr int kLds = kOffSeg + (APB_MAX_Q_HEADS + 2) * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
  uint8_t *const ring = smem;
  float *const sb1 = reinterpret_cast<float *>(smem + kOffB1);
  float *const sw2 = reinterpret_cast<float *>(smem + kOffW2);
  float(*const red)[kTok] = reinterpret_cast<float(*)[kTok]>(smem + kOffRed);
  int *const seg_off = reinterpret_cast<int *>(smem + kOffSeg);

  // Argument fields as locals.
  const uint16_t *const q = a.q, *const k = a.k, *const v = a.v;
  const float *const b1 = a.b1, *const w2 = a.w2, *const b2 = a.b2;
  float *const scores = a.scores;
  const int L = a.L, Hq = a.Hq, Hkv = a.Hkv, g = a.g, d = a.d, n_ttiles = a.n_ttiles;

  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int w = (bid % kNumXcd) * (nb / kNumXcd) + bid / kNumXcd;
  if (w >= n_ttiles * Hkv) return;
  const int h = w / n_ttiles;
  const int t0 = (w - h * n_ttiles) * kTok;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hq = wave & 3;   // hidden quarter
  const int th = wave >> 2;  // token half
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int din = (g + 2) * d;
  const int n_chunks = din / kKC;
  const int valid_rows = min(L - t0, kTok);
  const int q_row_bytes = Hq * d * 2;
  const int kv_row_bytes = Hkv * d * 2;
  // hidden = a.hidden <= HS: W1 rows past it read as zeros (the descriptor ends at
  // the last row), and their b1 and w2 are zero, so padded units add nothing.
  const int hidden = a.hidden;
  const uint16_t *w1h = a.w1 + (size_t)h * hidden * din;
  const int w_valid = hidden * din * 2;

  for (int i = tid; i < HS; i += kThreads) {
    sb1[i] = i < hidden ? b1[(size_t)h * hidden + i] : 0.f;
    sw2[i] = i < hidden ? w2[(size_t)h * hidden + i] : 0.f;
  }
  // Element offset of each x segment inside its tensor row: q heads of the group
  // (ascending), then k and v of head h.  The q-head table is read in place from
  // the kernel-argument segment into its own LDS array, read once per chunk.
#if defined(__HIP_DEVICE_COMPILE__)
  const uint8_t *qtab = (const uint8_t *)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(ScoreArgs, qhead_of_slot);
  for (int j = tid; j < g + 2; j += kThreads) seg_off[j] = (j < g ? (int)qtab[h * g + j] : h) * d;
#endif

  // ---- per-lane DMA offsets.  Load i covers rows i*8 .. i*8+7 of a chunk;
  // lane p writes bytes [16p, 16p+16): row i*8 + p/8, physical piece p%8, which
  // holds logical piece (p%8) ^ swz(row).
  const int pr = lane >> 3;
  const int pp = lane & 7;
  const int rx = wave * 32 + pr;  // rows of this wave's X loads: rx + 8i
  int xq[kXL], xkv[kXL];
#pragma unroll
  for (int i = 0; i < kXL; ++i) {
    const int r = rx + 8 * i;
    xq[i] = r * q_row_bytes + ((pp ^ swz(r)) * 16);
    xkv[i] = r * kv_row_bytes + ((pp ^ swz(r)) * 16);
  }
  // W1 load li, lane p: row li*8 + pr.  swz reads row bits 1..3; bit 3 is li's
  // low bit, which is the wave's (li = wave + NW*j with NW even).
  const int wrow = (wave & 1) * 8 + pr;
  const int wo_base = pr * din * 2 + ((pp ^ swz(wrow)) * 16);

  f32x16 acc[MBW][4];
#pragma unroll
  for (int j = 0; j < MBW; ++j)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[j][tb] = f32x16{};

  __syncthreads();  // seg_off, sb1, sw2 written

  const SrcCtx ctx{q + (size_t)t0 * Hq * d, k + (size_t)t0 * Hkv * d, v + (size_t)t0 * Hkv * d, w1h,
                   valid_rows * q_row_bytes, valid_rows * kv_row_bytes, xq, xkv, g, d};

  // ---- prologue: chunks 0 .. PF-1 in flight (PF = kRing - 1), chunk 0 landed
  constexpr int PF = kRing - 1;
  const int per_chunk = loads_per_chunk<WI_TOTAL, NW>(wave);
  const int n_pro = min(PF, n_chunks);
  for (int c = 0; c < n_pro; ++c)
    issue_chunk<WI_TOTAL, NW, kXB>(chunk_src(ctx, seg_off, c), ring + c * SLOT, w_valid, wo_base, din * 2, wave);
  wait_vmcnt_dyn((n_pro - 1) * per_chunk);
  barrier_keep_dma();

  // ---- main loop: chunk c in slot c % kRing; chunks c+1 .. c+PF-1 landed or
  // landing; chunk c+PF issued here into the slot chunk c-1 has freed.
  int slot = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if (c + PF < n_chunks) {
      const int sp = (slot + PF >= kRing) ? slot + PF - kRing : slot + PF;
      issue_chunk<WI_TOTAL, NW, kXB>(chunk_src(ctx, seg_off, c + PF), ring + sp * SLOT, w_valid, wo_base, din * 2,
                                     wave);
    }
    score_chunk<HB, kXB>(acc, ring + slot * SLOT, hq, th, lrow, half);
    // chunk c+1 must have landed; this wave's loads of chunks c+2 .. c+PF may stay in flight
    const int newer = min(PF, n_chunks - 1 - c) - 1;  // issued chunks after c+1
    if constexpr (WI_TOTAL % NW == 0) {
      if (newer == PF - 1) wait_vmcnt<(PF - 1) * (kXL + WI_TOTAL / NW)>();  // steady state
      else wait_vmcnt_dyn(newer > 0 ? newer * per_chunk : 0);
    } else {
      wait_vmcnt_dyn(newer > 0 ? newer * per_chunk : 0);
    }
    barrier_keep_dma();
    slot = (slot + 1 == kRing) ? 0 : slot + 1;
  }

  // ---- epilogue: lane holds hidden units mb*32 + 8*(i/4) + 4*half + i%4 of
  // tokens (th*4 + tb)*32 + lrow; partial w2 . relu(z + b1) per token, then
  // sum the four hidden quarters.
  // b1 and w2 of this lane's hidden units (the same for all four token blocks),
  // four consecutive units per 16-byte LDS read
  float4 b1v[MBW][4], w2v[MBW][4];
#pragma unroll
  for (int j = 0; j < MBW; ++j) {
    const int mb = hq + 4 * j;
    if (mb < HB) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int u0 = mb * 32 + q4 * 8 + half * 4;
        b1v[j][q4] = *reinterpret_cast<const float4 *>(sb1 + u0);
        w2v[j][q4] = *reinterpret_cast<const float4 *>(sw2 + u0);
      }
    }
  }
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < MBW; ++j) {
      const int mb = hq + 4 * j;
      if (mb < HB) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float bb = b1v[j][i >> 2][i & 3], ww = w2v[j][i >> 2][i & 3];
          part = fmaf(ww, fmaxf(acc[j][tb][i] + bb, 0.f), part);
        }
      }
    }
    part = half_swap_sum(part);
    if (half == 0) red[hq][(th * 4 + tb) * 32 + lrow] = part;
  }
  __syncthreads();
  if (tid < valid_rows) {
    const float sc = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid] + b2[h];
    scores[(size_t)h * L + t0 + tid] = sc;
  }
}

template <int HB>
hipError_t launch_hs(ScoreArgs &a, hipStream_t s) {
  using C = ScoreCfg<kTH>;
  a.n_ttiles = (a.L + C::kTok - 1) / C::kTok;
  const int n_work = a.n_ttiles * a.Hkv;
  const int grid = (n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL((score_kv_kernel<HB, kTH>), dim3(grid), dim3(C::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_kv(ScoreArgs &a, hipStream_t s) {
  switch ((a.hidden + 31) / 32) {
    case 1: return launch_hs<1>(a, s);
    case 2: return launch_hs<2>(a, s);
    case 3: return launch_hs<3>(a, s);
    case 4: return launch_hs<4>(a, s);
    case 5: return launch_hs<5>(a, s);
    case 6: return launch_hs<6>(a, s);
    case 7: return launch_hs<7>(a, s);
    default: return launch_hs<8>(a, s);
  }
}

}  // namespace apb
