// QKV projection of a host's hidden states, before the scoring step:
// q = x Wq^T, k = x Wk^T, v = x Wv^T (nn.Linear weights [out][in]).  The host's
// q, k and v feed every later step (juejin.cn APB explainer, section
// "APB 的主要功能": each host computes on its own block of the evenly split input).
//
// One kernel computes C[M][N] = X[M][K] W[N][K]^T in bf16 with fp32
// accumulation; three launches fill q, k and v.
//
// gfx950 design: a workgroup of 8 waves computes a 256 (tokens) x 256 (outputs)
// tile on v_mfma_f32_32x32x16_bf16 as C^T = W X^T (M of the MFMA = outputs,
// N = tokens), K walked in 32-wide chunks.  Wave w owns output blocks w%4 and
// w%4 + 4 (of 8 blocks of 32) for token half w/4 (four token blocks of 32):
// 8 accumulators of 32x32.  X and W chunks (16 KB each) reach LDS by LDS-DMA
// through a 3-slot ring (two chunks in flight while one is consumed); rows are
// 64 bytes with 16-byte pieces XOR-swizzled by row, so operand reads are free of
// bank conflicts.  Buffer descriptors end at the last valid row, so rows past M
// or N read as zeros and ragged tiles need no special path.  Consecutive work
// items on an XCD share an output slice, so its W rows stay in that XCD's L2
// while the token tiles stream by.  Each lane stores 4 consecutive outputs of
// one token (8 bytes) per accumulator group.
#include "lds_dma.h"

namespace apb {
namespace {

constexpr int kThreads = 512;   // 8 waves
constexpr int kNW = 8;
constexpr int kTile = 256;      // tokens and outputs per workgroup
constexpr int kKC = 32;         // K chunk
constexpr int kRowB = kKC * 2;  // 64 bytes per chunk row
constexpr int kXB = kTile * kRowB;   // 16 KB
constexpr int kWB = kTile * kRowB;   // 16 KB
constexpr int kSlot = kXB + kWB;
constexpr int kRing = 3;
constexpr int kPF = kRing - 1;

// Two fp32 values rounded to bf16 (nearest even), packed low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

// C^T[output block, token block] += W X^T for output quarter oq, token half th.
__device__ __forceinline__ void proj_chunk(f32x16 (&acc)[2][4], const uint8_t *__restrict__ cur, int oq, int th,
                                           int lrow, int half) {
  const uint8_t *ws = cur + kXB;
#pragma unroll
  for (int kk = 0; kk < kKC / 16; ++kk) {
    const int lp = 2 * kk + half;
    bf16x8 xf[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int r = (th * 4 + tb) * 32 + lrow;
      xf[tb] = *reinterpret_cast<const bf16x8 *>(cur + r * kRowB + ((lp ^ piece_swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = (oq + 4 * j) * 32 + lrow;
      const bf16x8 wf = *reinterpret_cast<const bf16x8 *>(ws + r * kRowB + ((lp ^ piece_swz(r)) * 16));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        acc[j][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[tb], acc[j][tb], 0, 0, 0);
    }
  }
}

// This wave's LDS-DMA loads of chunk c (p0 = 32c elements into every row): X rows
// wave*32 + {0, 16} + lane/4 and W rows of loads wave and wave + 8.
__device__ __forceinline__ void issue_proj_chunk(const uint16_t *x0, int x_valid,
                                                 const uint16_t *w0, int w_valid, int xo0, int xo1, int wo0,
                                                 int wo1, int p0, uint8_t *slot, int wave) {
  uint8_t *xd = slot + wave * 2 * 1024;
  dma_1k(x0 + p0, x_valid, xo0, xd);
  dma_1k(x0 + p0, x_valid, xo1, xd + 1024);
  dma_1k(w0 + p0, w_valid, wo0, slot + kXB + wave * 1024);
  dma_1k(w0 + p0, w_valid, wo1, slot + kXB + (wave + kNW) * 1024);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
void proj_gemm_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kRing * kSlot];

  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int w = (bid % kNumXcd) * (nb / kNumXcd) + bid / kNumXcd;
  if (w >= a.n_mt * a.n_nt) return;
  const int nt = w / a.n_mt;            // output slice: shared by consecutive work items
  const int mt = w - nt * a.n_mt;
  const int m0 = mt * kTile, n0 = nt * kTile;
  const int K = a.K;
  const int row_bytes = K * 2;
  const int x_rows = min(a.M - m0, kTile);
  const int w_rows = min(a.N - n0, kTile);
  const uint16_t *x0 = a.x + (size_t)m0 * K;
  const uint16_t *w0 = a.w + (size_t)n0 * K;
  const int x_valid = x_rows * row_bytes;   // rows past the end read as zeros
  const int w_valid = w_rows * row_bytes;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int oq = wave & 3;
  const int th = wave >> 2;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  // DMA lane offsets: load i covers chunk rows 16i .. 16i+15; lane p writes row
  // 16i + p/4, physical piece p%4, which holds logical piece (p%4) ^ swz(row).
  const int pr = lane >> 2;
  const int pp = lane & 3;
  const int rx = wave * 32 + pr;
  const int xo0 = rx * row_bytes + ((pp ^ piece_swz(rx)) * 16);
  const int xo1 = (rx + 16) * row_bytes + ((pp ^ piece_swz(rx + 16)) * 16);
  const int rw0 = wave * 16 + pr, rw1 = (wave + kNW) * 16 + pr;
  const int wo0 = rw0 * row_bytes + ((pp ^ piece_swz(rw0)) * 16);
  const int wo1 = rw1 * row_bytes + ((pp ^ piece_swz(rw1)) * 16);

  f32x16 acc[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[j][tb] = f32x16{};

  const int n_chunks = K / kKC;
  const int n_pro = min(kPF, n_chunks);
  for (int c = 0; c < n_pro; ++c)
    issue_proj_chunk(x0, x_valid, w0, w_valid, xo0, xo1, wo0, wo1, c * kKC, ring + c * kSlot, wave);
  wait_vmcnt_dyn((n_pro - 1) * 4);
  barrier_keep_dma();

  int slot = 0;
  for (int c = 0; c < n_chunks; ++c) {
    if (c + kPF < n_chunks) {
      const int sp = (slot + kPF >= kRing) ? slot + kPF - kRing : slot + kPF;
      issue_proj_chunk(x0, x_valid, w0, w_valid, xo0, xo1, wo0, wo1, (c + kPF) * kKC, ring + sp * kSlot, wave);
    }
    proj_chunk(acc, ring + slot * kSlot, oq, th, lrow, half);
    // chunk c+1 must have landed; this wave's 4 loads of each later chunk may stay in flight
    const int newer = min(kPF, n_chunks - 1 - c) - 1;
    if (newer == kPF - 1) wait_vmcnt<(kPF - 1) * 4>();
    else wait_vmcnt<0>();
    barrier_keep_dma();
    slot = (slot + 1 == kRing) ? 0 : slot + 1;
  }

  // ---- epilogue: lane holds outputs n0 + ob*32 + 8*(i/4) + 4*half + i%4 of token
  // m0 + (th*4 + tb)*32 + lrow; 4 consecutive outputs go out as one 8-byte store.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ob = oq + 4 * j;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int m = (th * 4 + tb) * 32 + lrow;
      if (m >= x_rows) continue;
      uint16_t *crow = a.c + (size_t)(m0 + m) * a.N + n0;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int n = ob * 32 + g4 * 8 + half * 4;
        if (n >= w_rows) continue;
        uint2 p;
        p.x = pack_bf16x2(acc[j][tb][g4 * 4 + 0], acc[j][tb][g4 * 4 + 1]);
        p.y = pack_bf16x2(acc[j][tb][g4 * 4 + 2], acc[j][tb][g4 * 4 + 3]);
        *reinterpret_cast<uint2 *>(crow + n) = p;
      }
    }
  }
}

}  // namespace

hipError_t launch_proj_gemm(ProjArgs &a, hipStream_t s) {
  a.n_mt = (a.M + kTile - 1) / kTile;
  a.n_nt = (a.N + kTile - 1) / kTile;
  const int n_work = a.n_mt * a.n_nt;
  const int grid = (n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
