// APB step 1: per-kv-head importance score of each local token.
//
// Stand-in for Locret's retaining heads (juejin.cn APB explainer, section
// "APB 的主要功能": each host compresses its KV cache with retaining heads;
// section "APB 的技术原理": the query sits at the start of the anchor so the
// compressor sees it).  For kv head h and token t:
//   x = [q[t, G_h[0]]; ...; q[t, G_h[g-1]]; k[t, h]; v[t, h]]
//   s = w2[h] . relu(W1[h] x + b1[h]) + b2[h]
//
// gfx950 design: Z^T = W1 X^T on v_mfma_f32_32x32x16_bf16 (M = hidden units,
// N = tokens, K = (g+2)d).  Each wave owns 32 tokens and every hidden unit, so
// the ReLU and the w2 dot product finish inside the wave (one lane-half swap).
// X is streamed from HBM straight into B-operand registers (each byte is read
// exactly once), prefetched one 64-wide K chunk ahead; W1 chunks are staged in
// double-buffered LDS and shared by the workgroup's 4 waves.  Work items are
// grouped by kv head onto XCDs so a head's W1 stays in one L2.
#include "apb_internal.h"

namespace apb {
namespace {

constexpr int kThreads = 256;
constexpr int kTok = 128;      // tokens per workgroup (4 waves x 32)
constexpr int kKC = 64;        // K chunk (elements of x)
constexpr int kWP = kKC + 8;   // W1 LDS row pitch in u16

__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int HSB>  // hidden = 32 * HSB
__global__ __launch_bounds__(kThreads) void score_kv_kernel(const ScoreArgs a) {
  constexpr int HS = 32 * HSB;
  constexpr int WCH = HS * kKC / 8;                 // 16-byte pieces per W1 chunk
  constexpr int WIT = (WCH + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t wbuf[2][HS * kWP];

  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int w = (bid % kNumXcd) * (nb / kNumXcd) + bid / kNumXcd;
  const int n_work = a.n_ttiles * a.Hkv;
  if (w >= n_work) return;
  const int h = w / a.n_ttiles;
  const int tt = w - h * a.n_ttiles;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lrow = lane & 31;
  const int half = lane >> 5;
  const int d = a.d;
  const int din = (a.g + 2) * d;
  const int n_chunks = din / kKC;
  const int tok = tt * kTok + wave * 32 + lrow;
  const bool tok_ok = tok < a.L;
  const uint16_t *w1h = a.w1 + (size_t)h * HS * din;

  // Address of x[tok][p .. p+7] for p a multiple of 8.
  auto x_ptr = [&](int p) -> const uint16_t * {
    const int seg = p / d;
    const int off = p - seg * d;
    if (seg < a.g) return a.q + (size_t)tok * a.Hq * d + a.qhead_of_slot[h * a.g + seg] * d + off;
    if (seg == a.g) return a.k + (size_t)tok * a.Hkv * d + h * d + off;
    return a.v + (size_t)tok * a.Hkv * d + h * d + off;
  };

  auto load_x = [&](int c, bf16x8 (&xf)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (tok_ok) xf[kk] = *reinterpret_cast<const bf16x8 *>(x_ptr(c * kKC + kk * 16 + half * 8));
      else xf[kk] = bf16x8{};
    }
  };

  uint4 wreg[WIT];
  auto load_w = [&](int c) {
#pragma unroll
    for (int it = 0; it < WIT; ++it) {
      const int piece = it * kThreads + tid;
      if (piece < WCH) {
        const int row = piece / (kKC / 8);
        const int col = piece % (kKC / 8);
        wreg[it] = *reinterpret_cast<const uint4 *>(w1h + (size_t)row * din + c * kKC + col * 8);
      }
    }
  };
  auto store_w = [&](uint16_t *buf) {
#pragma unroll
    for (int it = 0; it < WIT; ++it) {
      const int piece = it * kThreads + tid;
      if (piece < WCH) {
        const int row = piece / (kKC / 8);
        const int col = piece % (kKC / 8);
        *reinterpret_cast<uint4 *>(buf + row * kWP + col * 8) = wreg[it];
      }
    }
  };

  f32x16 acc[HSB];
#pragma unroll
  for (int mb = 0; mb < HSB; ++mb) acc[mb] = f32x16{};

  bf16x8 xcur[4], xnext[4];
  load_x(0, xcur);
  load_w(0);
  store_w(wbuf[0]);
  __syncthreads();

  for (int c = 0; c < n_chunks; ++c) {
    if (c + 1 < n_chunks) {
      load_x(c + 1, xnext);
      load_w(c + 1);
    }
    const uint16_t *wb = wbuf[c & 1];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int mb = 0; mb < HSB; ++mb) {
        const bf16x8 wf = *reinterpret_cast<const bf16x8 *>(wb + (mb * 32 + lrow) * kWP + kk * 16 + half * 8);
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xcur[kk], acc[mb], 0, 0, 0);
      }
    }
    if (c + 1 < n_chunks) {
      store_w(wbuf[(c + 1) & 1]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) xcur[kk] = xnext[kk];
    }
    __syncthreads();
  }

  // Epilogue: lane holds hidden units mb*32 + 8*(i/4) + 4*half + i%4 of token `tok`.
  const float *b1h = a.b1 + (size_t)h * HS;
  const float *w2h = a.w2 + (size_t)h * HS;
  float part = 0.f;
#pragma unroll
  for (int mb = 0; mb < HSB; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = mb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
      part = fmaf(w2h[u], fmaxf(acc[mb][i] + b1h[u], 0.f), part);
    }
  }
  const float tot = half_swap_sum(part) + a.b2[h];
  if (tok_ok && half == 0) a.scores[(size_t)h * a.L + tok] = tot;
}

template <int HSB>
hipError_t launch_hs(ScoreArgs &a, hipStream_t s) {
  a.n_ttiles = (a.L + kTok - 1) / kTok;
  const int n_work = a.n_ttiles * a.Hkv;
  const int grid = (n_work + kNumXcd - 1) / kNumXcd * kNumXcd;
  hipLaunchKernelGGL((score_kv_kernel<HSB>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_score_kv(ScoreArgs &a, hipStream_t s) {
  switch (a.hidden / 32) {
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
