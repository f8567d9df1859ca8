// QKV projection of a host's hidden states, before the scoring step:
// q = x Wq^T, k = x Wk^T, v = x Wv^T (nn.Linear weights [out][in]).  The host's
// q, k and v feed every later step (juejin.cn APB explainer, section
// "APB 的主要功能": each host computes on its own block of the evenly split input).
//
// One launch computes all three: C[M][N] = X[M][K] W[N][K]^T in bf16 with fp32
// accumulation, the output columns of q, k and v cut into 256-wide slices that
// form one work list.
//
// gfx950 design.  A workgroup of 4 waves (one per SIMD) computes a 256 (tokens)
// x 256 (outputs) tile on v_mfma_f32_32x32x16_bf16 as C^T = W X^T (M of the
// MFMA = outputs, N = tokens).  Wave w owns token half w/2 and output half w%2:
// 4 x 4 accumulators of 32x32, 256 accumulator registers.  K is walked in
// 64-wide chunks; X and W chunks (32 KB each) reach LDS by LDS-DMA through two
// 64 KB slots, one chunk in flight while the other is consumed:
//  * each wave's 16 DMA loads of the next chunk are interleaved with its first
//    32 MFMAs of the current one, so the single wave per SIMD never stops
//    issuing MFMAs to issue loads;
//  * a chunk's last K step is multiplied after the barrier that ends the chunk
//    (its operands are already in registers), covering the latency of the next
//    chunk's first LDS reads;
//  * 128-byte chunk rows hold 16-byte pieces XOR-swizzled by row, so the 16
//    lanes of each LDS read cycle hit 16 distinct bank groups.
// Buffer descriptors end at the tile's last valid byte, so rows past M or N
// read as zeros and ragged tiles need no special path; K % 64 == 32 adds one
// half chunk.  Work items go in groups of 8 token tiles x all output slices,
// token tile fastest, so the workgroups resident on one XCD at a time share a
// few X tiles and a few W slices through that XCD's L2.  The finished tile is
// rounded to bf16 into the (by then idle) LDS ring and leaves in whole 512-byte
// rows, 16 bytes per lane: stored straight from the accumulators, each store
// instruction wrote 8 bytes into each of 32 rows, and that epilogue took about
// an eighth of a workgroup's time.
#include "lds_dma.h"

namespace apb {
namespace {

constexpr int kNW = 4;                  // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kTile = 256;              // tokens and outputs per workgroup
constexpr int kKC = 64;                 // K chunk
constexpr int kRowB = kKC * 2;          // 128 bytes per chunk row
constexpr int kPPR = kKC / 8;           // 8 pieces of 16 bytes per row
constexpr int kRPI = 64 / kPPR;         // 8 rows per 1 KB DMA load
constexpr int kOpB = kTile * kRowB;     // 32 KB: one operand's chunk
constexpr int kSlot = 2 * kOpB;         // X chunk, then W chunk
constexpr int kLoads = kTile / kRPI / kNW;   // 8 DMA loads per wave per operand
constexpr int kPerChunk = 2 * kLoads;        // 16 per wave per chunk
constexpr int kHalfLoads = kPerChunk / 2;
constexpr int kOutB = 4;                // 32-wide output blocks per wave
constexpr int kMfma = kOutB * 4;        // MFMAs per 16-wide K step
constexpr int kReads = 4 + kOutB;       // LDS reads per K step
constexpr int kKK = kKC / 16;           // K steps per chunk
constexpr int kGroupM = 8;              // token tiles per work-item group
constexpr int kOutRowB = kTile * 2;     // 512 bytes: one token's bf16 outputs in the staged tile
static_assert(kTile * kOutRowB <= 2 * kSlot, "the staged output tile fits in the LDS ring");
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte piece p of chunk row r sits at piece p ^ swz(r): rows r .. r+15 of
// one read cycle cover all 16 (row parity, piece) bank groups of 256 bytes.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Two fp32 values rounded to bf16 (nearest even), packed low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p;
  p[0] = (__bf16)a;
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}

// Operand fragments of one 16-wide K step: four token blocks, four output blocks.
struct ProjFrags {
  bf16x8 x[4];
  bf16x8 w[kOutB];
};

// Per-lane LDS byte offsets, within a slot, of this lane's rows at K step 0:
// row*128 + (half ^ swz(row))*16.  Step kk reads offset ^ (kk << 5): the XOR
// flips only the piece bits, so piece 2kk + half lands on physical piece
// (2kk + half) ^ swz(row).
struct ProjLanes {
  int x[4];
  int w[kOutB];
};

// slot_off (a multiple of the slot size) changes from chunk to chunk, so the
// per-step offsets are recomputed (one XOR each) rather than hoisted into
// registers beside the accumulators.
__device__ __forceinline__ void load_frags(ProjFrags &f, const uint8_t *__restrict__ ring, int slot_off,
                                           const ProjLanes &ln, int kk) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
    f.x[tb] = *reinterpret_cast<const bf16x8 *>(ring + ((slot_off + ln.x[tb]) ^ (kk << 5)));
#pragma unroll
  for (int j = 0; j < kOutB; ++j)
    f.w[j] = *reinterpret_cast<const bf16x8 *>(ring + ((slot_off + ln.w[j]) ^ (kk << 5)));
}

__device__ __forceinline__ void mfma_step(f32x16 (&acc)[kOutB][4], const ProjFrags &g) {
#pragma unroll
  for (int j = 0; j < kOutB; ++j)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      acc[j][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(g.w[j], g.x[tb], acc[j][tb], 0, 0, 0);
}

// Loads Q0 .. Q1-1 of this wave's share of the chunk that starts p0 elements
// into every row (loads below kLoads are X, the rest W).  Load i of an operand
// (i = wave*kLoads + j) fills rows 8i .. 8i+7 of its chunk.  The ranges are the
// bytes left in the tile from the chunk's base, so they end at the tile's last
// valid byte; a zero range makes the loads no-ops that touch no memory.
template <int Q0, int Q1>
__device__ __forceinline__ void issue_part(const uint16_t *x0, int x_range, const uint16_t *w0, int w_range,
                                           const int (&off)[kLoads], int p0, uint8_t *slot, int wave) {
#pragma unroll
  for (int q = Q0; q < Q1; ++q) {
    if (q < kLoads)
      dma_1k(x0 + p0, x_range, off[q], slot + (wave * kLoads + q) * 1024);
    else
      dma_1k(w0 + p0, w_range, off[q - kLoads], slot + kOpB + (wave * kLoads + q - kLoads) * 1024);
  }
}

// Scheduling hints: N pairs of (M MFMAs, one instruction of class MASK).
template <int N, int M, int MASK>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
    __builtin_amdgcn_sched_group_barrier(MASK, 1, 0);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void proj_gemm_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[2 * kSlot];

  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int w = (bid % kNumXcd) * (nb / kNumXcd) + bid / kNumXcd;
  if (w >= a.n_mt * a.n_nt) return;
  const int per_group = kGroupM * a.n_nt;
  const int gid = w / per_group;
  const int first_m = gid * kGroupM;
  const int gsize = min(a.n_mt - first_m, kGroupM);
  const int wr = w - gid * per_group;
  const int mt = first_m + wr % gsize;
  const int nt = wr / gsize;
  // which of q, k, v the slice belongs to (wave-uniform selects, no indexing)
  const int mat = nt < a.slice_end[0] ? 0 : (nt < a.slice_end[1] ? 1 : 2);
  const int ns = nt - (mat == 0 ? 0 : (mat == 1 ? a.slice_end[0] : a.slice_end[1]));
  const uint16_t *wmat = mat == 0 ? a.w[0] : (mat == 1 ? a.w[1] : a.w[2]);
  uint16_t *cmat = mat == 0 ? a.c[0] : (mat == 1 ? a.c[1] : a.c[2]);
  const int N = mat == 0 ? a.N[0] : (mat == 1 ? a.N[1] : a.N[2]);

  const int m0 = mt * kTile, n0 = ns * kTile;
  const int K = a.K;
  const int row_bytes = K * 2;
  const int x_rows = min(a.M - m0, kTile);
  const int w_rows = min(N - n0, kTile);
  const uint16_t *x0 = a.x + (size_t)m0 * K;
  const uint16_t *w0 = wmat + (size_t)n0 * K;
  const int x_bytes = x_rows * row_bytes;   // rows past the end read as zeros
  const int w_bytes = w_rows * row_bytes;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int oh = wave & 1;                  // output half: blocks 4*oh .. 4*oh+3
  const int th = wave >> 1;                 // token half: blocks 4*th .. 4*th+3
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  // DMA lane offsets (the same for X and W): lane p writes row 8i + p/8,
  // physical piece p%8, which holds logical piece (p%8) ^ swz(row).
  const int pr = lane / kPPR;
  const int pp = lane % kPPR;
  int off[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const int r = (wave * kLoads + j) * kRPI + pr;
    off[j] = r * row_bytes + ((pp ^ swz(r)) * 16);
  }
  ProjLanes ln;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int r = (th * 4 + tb) * 32 + lrow;
    ln.x[tb] = r * kRowB + ((half ^ swz(r)) * 16);
  }
#pragma unroll
  for (int j = 0; j < kOutB; ++j) {
    const int r = (oh * 4 + j) * 32 + lrow;
    ln.w[j] = kOpB + r * kRowB + ((half ^ swz(r)) * 16);
  }

  f32x16 acc[kOutB][4];
#pragma unroll
  for (int j = 0; j < kOutB; ++j)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[j][tb] = f32x16{};

  const int n_full = K / kKC;
  const int n_chunks = (K + kKC - 1) / kKC;    // K % 32 == 0: a tail is half a chunk
  issue_part<0, kPerChunk>(x0, x_bytes, w0, w_bytes, off, 0, ring, wave);
  wait_vmcnt<0>();
  barrier_lds_drained();

  // The last K step of each chunk is multiplied after the barrier that ends the
  // chunk: its fragments are already in registers (the barrier drains LDS
  // reads), and its MFMAs cover the latency of the next chunk's first reads.
  ProjFrags hold, nxt;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) hold.x[tb] = bf16x8{};
#pragma unroll
  for (int j = 0; j < kOutB; ++j) hold.w[j] = bf16x8{};
  int slot = 0;
  if (n_full > 0) load_frags(nxt, ring, 0, ln, 0);
  for (int c = 0; c < n_full; ++c) {
    // Chunk c+1 goes into the other slot, which held chunk c-1 and which every
    // wave has finished reading; past the last chunk the loads get a zero range.
    const bool live = c + 1 < n_chunks;
    const int pf = (c + 1) * kKC;
    const int xr = live ? x_bytes - 2 * pf : 0;
    const int wrg = live ? w_bytes - 2 * pf : 0;
    uint8_t *sdst = ring + (slot ^ 1) * kSlot;
    issue_part<0, kHalfLoads>(x0, xr, w0, wrg, off, pf, sdst, wave);
    mfma_step(acc, hold);   // zero operands on the first chunk
    interleave<kHalfLoads, kMfma / kHalfLoads, 0x020>();
    __builtin_amdgcn_sched_barrier(0);
    ProjFrags f = nxt;
#pragma unroll
    for (int kk = 0; kk + 1 < kKK; ++kk) {
      ProjFrags g;
      load_frags(g, ring, slot * kSlot, ln, kk + 1);
      if (kk == 0) issue_part<kHalfLoads, kPerChunk>(x0, xr, w0, wrg, off, pf, sdst, wave);
      mfma_step(acc, f);
      interleave<kReads, 1, 0x100>();
      if (kk == 0) interleave<kHalfLoads, 1, 0x020>();
      __builtin_amdgcn_sched_barrier(0);
      f = g;
    }
    hold = f;
    wait_vmcnt<0>();          // this wave's loads of chunk c+1 have landed
    barrier_lds_drained();    // everyone's have, and chunk c is read
    slot ^= 1;
    if (c + 1 < n_full) load_frags(nxt, ring, slot * kSlot, ln, 0);
  }
  mfma_step(acc, hold);
  // The half chunk (K % 64 == 32) landed before the last barrier.
  if (n_chunks > n_full) {
    ProjFrags f, g;
    load_frags(f, ring, slot * kSlot, ln, 0);
    load_frags(g, ring, slot * kSlot, ln, 1);
    mfma_step(acc, f);
    mfma_step(acc, g);
  }

  // ---- epilogue: the tile goes to LDS as bf16 (256 rows of 512 bytes, 16-byte
  // pieces XOR-swizzled by row), then out in whole 512-byte rows.
  barrier_lds_drained();    // every wave has read its last fragments from the ring
  // Lane: token row (th*4 + tb)*32 + lrow, outputs ob*32 + 8*g4 + 4*half .. +3,
  // i.e. half of 16-byte piece ob*4 + g4 of that row.
#pragma unroll
  for (int j = 0; j < kOutB; ++j) {
    const int ob = oh * 4 + j;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int m = (th * 4 + tb) * 32 + lrow;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int piece = ob * 4 + g4;
        uint2 p;
        p.x = pack_bf16x2(acc[j][tb][g4 * 4 + 0], acc[j][tb][g4 * 4 + 1]);
        p.y = pack_bf16x2(acc[j][tb][g4 * 4 + 2], acc[j][tb][g4 * 4 + 3]);
        *reinterpret_cast<uint2 *>(ring + m * kOutRowB + ((piece ^ (m & 31)) << 4) + half * 8) = p;
      }
    }
  }
  barrier_lds_drained();
  // Thread t writes piece t % 32 of row 8i + t / 32: two whole rows per wave.
  const int piece = tid & 31;
  const bool col_ok = piece * 8 < w_rows;   // w_rows is a multiple of 64
#pragma unroll 4
  for (int i = 0; i < kTile / (kThreads / 32); ++i) {
    const int row = i * (kThreads / 32) + (tid >> 5);
    if (row >= x_rows || !col_ok) continue;
    const u32x4 val = *reinterpret_cast<const u32x4 *>(ring + row * kOutRowB + ((piece ^ (row & 31)) << 4));
    *reinterpret_cast<u32x4 *>(cmat + (size_t)(m0 + row) * N + n0 + piece * 8) = val;
  }
}

}  // namespace

hipError_t launch_proj_gemm(ProjArgs &a, hipStream_t s) {
  // the epilogue writes whole 16-byte pieces of output rows
  for (int i = 0; i < 3; ++i)
    if (a.N[i] < 64 || a.N[i] % 64 != 0) return hipErrorInvalidValue;
  a.n_mt = (a.M + kTile - 1) / kTile;
  int end = 0;
  for (int i = 0; i < 3; ++i) {
    end += (a.N[i] + kTile - 1) / kTile;
    a.slice_end[i] = end;
  }
  a.n_nt = end;
  const int n_work = a.n_mt * a.n_nt;
  const int grid = (n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL(proj_gemm_kernel, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace apb
