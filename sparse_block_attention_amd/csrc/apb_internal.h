// Internal declarations shared by the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apb.h"

namespace apb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Number of XCDs on MI355X; workgroups are dispatched to them round-robin.
constexpr int kNumXcd = 8;

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave stay
// outstanding.  The builtin (not inline asm) lets the compiler see the wait, so
// it knows which loads have landed.  gfx9 immediate: vmcnt in bits 3:0 and
// 15:14; expcnt (bits 6:4) and lgkmcnt (bits 11:8) at their maximum, i.e. not
// waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that leaves LDS-DMA loads in flight.  __syncthreads() is
// also a workgroup memory fence, for which the compiler drains every outstanding
// vector-memory operation, including prefetches meant to stay in flight across
// the barrier.  Callers wait (wait_vmcnt) for exactly the LDS-DMA data they
// need before this barrier; the barrier itself drains this wave's LDS reads,
// so a buffer everyone has finished reading may be overwritten after it.
__device__ __forceinline__ void barrier_keep_dma() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The same barrier built from compiler builtins (s_waitcnt lgkmcnt(0), then
// s_barrier): the compiler then knows this wave's LDS reads have landed and adds
// no wait of its own before later uses of their results.
__device__ __forceinline__ void barrier_lds_drained() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maximum (no wait)
  __builtin_amdgcn_s_barrier();
}

// Attention over [anchor | passing | local causal].
struct AttnArgs {
  const uint16_t *q, *ka, *va, *kp, *vp, *kl, *vl;
  uint16_t *out;
  float *lse;               // may be null
  int L, A, P, Hq, Hkv, g;  // A, P: rows of the anchor / passing segments attended (0 = left out)
  int use_local;            // 1: local rows 0..r are attended; 0: local segment left out
  int n_qtiles;             // ceil(L / rows per workgroup)
  int n_work;               // n_qtiles * Hq
  float scale_log2;         // softmax scale * log2(e)
  uint8_t qhead_of_slot[256];  // slot h*g + j -> j-th q head (ascending) of kv head h
};
hipError_t launch_block_attention(AttnArgs &a, int head_dim, hipStream_t s);

// Merge of two partial attention results over disjoint key sets.
struct MergeArgs {
  const uint16_t *oa, *ob;
  const float *la, *lb;
  uint16_t *out;
  float *lse;               // may be null
  int L, Hq, d;
};
hipError_t launch_merge_attention(const MergeArgs &a, hipStream_t s);

// C[M][N] = X[M][K] W[N][K]^T in bf16, fp32 accumulation (QKV projection).
// One launch covers the three weight matrices (q, k, v); their 256-wide output
// slices are numbered one after another.
struct ProjArgs {
  const uint16_t *x;
  const uint16_t *w[3];
  uint16_t *c[3];
  int N[3];                 // outputs of each matrix (heads x head_dim), N % 64 == 0
  int M, K;                 // K % 32 == 0
  int n_mt, n_nt;           // tiles of 256 along M; slices of 256 over all three N
  int slice_end[3];         // cumulative slice counts
};
hipError_t launch_proj_gemm(ProjArgs &a, hipStream_t s);

// Rotary position embedding (rotate-half pairing).
struct RopeArgs {
  const uint16_t *x;
  uint16_t *out;
  long long pos0;
  int rows, heads, d;
  double theta[64];         // theta_i = base^(-2i/d), i < d/2
};
hipError_t launch_rope(const RopeArgs &a, hipStream_t s);

// Scorer: per kv head, 2-layer ReLU MLP over [q of the group; k; v].
struct ScoreArgs {
  const uint16_t *q, *k, *v, *w1;
  const float *b1, *w2, *b2;
  float *scores;
  int L, Hq, Hkv, g, d, hidden;
  int n_ttiles;             // ceil(L / tokens per workgroup)
  uint8_t qhead_of_slot[256];
};
hipError_t launch_score_kv(ScoreArgs &a, hipStream_t s);

// Top-l selection + gather.  The workspace holds, per kv head, the selection
// state {T, need} and, per chunk of 256 keys, the counts of keys > T and == T in
// the chunks before it.
struct TopkArgs {
  const float *scores;
  const uint16_t *k, *v;
  int32_t *idx;
  uint16_t *kc, *vc;
  uint32_t *state;          // [Hkv][2]            (workspace)
  uint32_t *chunk_counts;   // [Hkv][n_chunks][2]  (workspace)
  int L, l, Hkv, d;
  int n_chunks;             // ceil(L / 256)
};
size_t topk_workspace_bytes(int L, int Hkv);
hipError_t launch_topk_gather(TopkArgs &a, void *workspace, hipStream_t s);

// Size of the per-GPU static workspace of apb_topk_gather_noalloc, and its device
// address on the current device (looked up once per device).
constexpr size_t kStaticTopkScratchBytes = APB_NOALLOC_TOPK_WORKSPACE_BYTES;
hipError_t static_topk_scratch(void **ptr);

// Passing-block assembly: up to 128 source blocks per launch.
struct PassArgs {
  const uint16_t *ksrc[128];
  const uint16_t *vsrc[128];
  uint16_t *kdst, *vdst;
  long long block_u16x8;    // 16-byte units per compressed block (l * Hkv * d / 8)
  int n_src;
};
hipError_t launch_build_passing(const PassArgs &a, hipStream_t s);

}  // namespace apb
