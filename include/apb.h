/*
 * apb.h - C ABI of the APB per-host prefill path on AMD MI355X (gfx950).
 *
 * APB ("Accelerating Distributed Long-Context Inference by Passing Compressed
 * Context Blocks across GPUs") splits a long prompt evenly over hosts.  One
 * host's share of one layer is four steps, each an entry point below:
 *
 *   apb_score_kv         score every local token per kv head (stand-in for
 *                        Locret's retaining heads);
 *   apb_topk_gather      keep the l best tokens per kv head and gather their
 *                        K/V rows: the host's compressed context block;
 *   apb_build_passing    concatenate the compressed blocks of the preceding
 *                        hosts: the passing block;
 *   apb_block_attention  attention of the local queries over
 *                        [anchor | passing | local, causal].
 *
 * apb_block_attention_segments and apb_merge_attention compute step 4 in parts
 * (anchor + local first, passing once it has arrived) and merge the parts.
 *
 * The steps are described on the juejin.cn explainer of APB, sections
 * "APB 的主要功能" (main functions) and "APB 的技术原理" (technical principles),
 * and in the paper's arXiv abstract (mlsanity.com/paper/2502.12085).
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned, contiguous, row-major DEVICE buffers, token
 *     major: [rows][heads][head_dim].  bf16 tensors are passed as void*.
 *     Every tensor pointer must be 16-byte aligned.  Outputs must not alias
 *     inputs (apb_merge_attention may write in place, see there).  The library
 *     allocates no device memory and keeps no state
 *     between calls other than a per-process cache of device properties.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous on that stream, reentrant and deterministic
 *     (identical inputs give identical output bits; no result depends on the
 *     order of atomic operations).
 *   - Arguments are checked on the host before anything is launched; a bad
 *     argument returns an error code and launches nothing.  A launch failure
 *     returns APB_ERR_HIP.  Faults inside a kernel surface at the caller's
 *     next synchronisation, as in HIP.  No call aborts, exits or throws;
 *     apb_last_error() gives a message for the calling thread's last error.
 */
#ifndef APB_H
#define APB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define APB_ABI_VERSION 5

/* Upper limits of this implementation (APB_ERR_UNSUPPORTED beyond them). */
#define APB_MAX_Q_HEADS 256
#define APB_MAX_LOCAL_LEN (1 << 26)
#define APB_MAX_PASS_HOSTS_PER_LAUNCH 128
#define APB_MAX_ROPE_POSITION (1LL << 31) /* apb_rope: pos0 + rows <= this */

typedef enum {
  APB_OK = 0,
  APB_ERR_INVALID_ARGUMENT = 1,    /* NULL / misaligned pointer, inconsistent sizes */
  APB_ERR_UNSUPPORTED = 2,         /* valid in principle, outside this library's limits */
  APB_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below apb_topk_workspace_size() */
  APB_ERR_HIP = 4,                 /* the HIP runtime reported an error */
  APB_ERR_INTERNAL = 5             /* unexpected failure inside the library */
} apb_status;

/*
 * One host's share of the split sequence (explainer, "APB 的主要功能": the
 * input is distributed evenly over hosts, an anchor block holding the start of
 * the sequence is prepended to each local block, and the passing block carries
 * the important KV of the preceding hosts).  Host memory, read during the call.
 */
typedef struct {
  int32_t n_q_heads;       /* Hq, 1..APB_MAX_Q_HEADS, a multiple of n_kv_heads       */
  int32_t n_kv_heads;      /* Hkv >= 1; g = Hq / Hkv q heads share one kv head      */
  int32_t head_dim;        /* d: 64 or 128                                           */
  int32_t local_len;       /* L: tokens in this host's block, 1..APB_MAX_LOCAL_LEN  */
  int32_t anchor_len;      /* A >= 0: anchor rows (the first A tokens of the sequence) */
  int32_t pass_per_host;   /* l: tokens kept per kv head per host, 0 <= l <= L       */
  int32_t host_index;      /* p: this host, 0 <= p < n_hosts; passing has P = p*l rows */
  int32_t n_hosts;         /* H >= 1                                                  */
  const int32_t *kv_head_of_q; /* host array [Hq] mapping q head -> kv head, or NULL
                                  for i -> i / g.  Each kv head must get exactly g q
                                  heads; a kv head's group is taken in ascending
                                  q-head order.                                      */
} apb_problem;

/*
 * Per-kv-head 2-layer scorer standing in for Locret's retaining heads
 * (explainer, "APB 的主要功能": each host compresses its KV cache with retaining
 * heads; "APB 的技术原理": the query sits at the start of the anchor so the
 * compressor sees it).  For kv head h and token t:
 *     x = [q[t, G_h[0]]; ...; q[t, G_h[g-1]]; k[t, h]; v[t, h]]   ((g+2)*d values)
 *     s = w2[h] . relu(W1[h] x + b1[h]) + b2[h]
 * Device pointers.  Products of bf16 values are accumulated in fp32.
 */
typedef struct {
  int32_t hidden;          /* Hs: a multiple of 16, 16..256                    */
  const void *w1;          /* bf16 [Hkv][Hs][(g+2)*d]  (nn.Linear weight layout) */
  const float *b1;         /* fp32 [Hkv][Hs]                                    */
  const float *w2;         /* fp32 [Hkv][Hs]                                    */
  const float *b2;         /* fp32 [Hkv]                                        */
} apb_scorer;

/*
 * Step 1: importance score of every local token, per kv head.
 *   q_local  bf16 [L][Hq][d]      k_local, v_local  bf16 [L][Hkv][d]
 *   scores   fp32 [Hkv][L]        (output)
 */
apb_status apb_score_kv(const apb_problem *problem, const apb_scorer *scorer,
                        const void *q_local, const void *k_local, const void *v_local,
                        float *scores, void *stream);

/*
 * Step 2: per kv head, keep the l highest scores and gather their K/V rows
 * into the compressed context block (explainer, "APB 的主要功能", compression
 * with retaining heads and the communication of the compressed blocks).
 * Order: larger fp32 score first; -0 equals +0; NaN ranks below every number
 * (including -inf); equal scores go to the lower token index.
 *   scores          fp32 [Hkv][L]
 *   k_local, v_local bf16 [L][Hkv][d]
 *   idx             int32 [Hkv][l] (output) selected local token indices, ascending
 *   k_comp, v_comp  bf16 [l][Hkv][d] (output) k_comp[s][h] = k_local[idx[h][s]][h]
 *   workspace       device scratch of at least apb_topk_workspace_size(problem)
 *                   bytes, 16-byte aligned, owned by the caller.  Its contents on
 *                   entry do not matter (every byte the call reads, it wrote
 *                   earlier in the same call) and are meaningless afterwards; two
 *                   calls in flight at once need two workspaces.
 * With l == 0 nothing is written and every pointer may be NULL.  A workspace
 * smaller than required returns APB_ERR_WORKSPACE_TOO_SMALL and launches nothing.
 */
/*
 * Bytes of workspace apb_topk_gather needs for `problem` (a few bytes per kv
 * head plus 8 bytes per 256 local tokens per kv head).  Returns 0 when the
 * problem is invalid (apb_last_error() says why) or when l == 0, where the
 * call does nothing and needs no workspace.  Host-only; launches nothing.
 */
size_t apb_topk_workspace_size(const apb_problem *problem);
apb_status apb_topk_gather(const apb_problem *problem, const float *scores,
                           const void *k_local, const void *v_local,
                           int32_t *idx, void *k_comp, void *v_comp,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * apb_topk_gather for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same selection and gather, same outputs, with the workspace taken from a
 * static array of APB_NOALLOC_TOPK_WORKSPACE_BYTES per GPU that the library
 * holds until the process ends, instead of a caller buffer.  The call allocates
 * nothing.  Problems whose workspace (apb_topk_workspace_size) exceeds that
 * size return APB_ERR_UNSUPPORTED and launch nothing.  Every call on one GPU
 * shares that GPU's array, so two calls whose kernels may overlap on one GPU
 * (different streams, no ordering between them) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the array has to
 * start at zero.
 */
#define APB_NOALLOC_TOPK_WORKSPACE_BYTES ((size_t)4 << 20)
apb_status apb_topk_gather_noalloc(const apb_problem *problem, const float *scores,
                                   const void *k_local, const void *v_local,
                                   int32_t *idx, void *k_comp, void *v_comp, void *stream);

/*
 * Step 3: passing block from the compressed blocks of hosts 0..p-1 (explainer,
 * "APB 的主要功能": the all-gathered compressed blocks form the passing block of
 * the preceding hosts' important KV; "APB 的技术原理": each block is compressed
 * and sent to the later GPUs).  Host-major: row j*l + s holds slot s of host j.
 *   k_comp_hosts, v_comp_hosts  HOST arrays of p device pointers, each bf16 [l][Hkv][d]
 *   k_pass, v_pass              bf16 [p*l][Hkv][d] (output)
 * With P == 0 nothing is written and every pointer may be NULL.
 */
apb_status apb_build_passing(const apb_problem *problem,
                             const void *const *k_comp_hosts, const void *const *v_comp_hosts,
                             void *k_pass, void *v_pass, void *stream);

/*
 * Step 4: attention of the local queries (explainer, "APB 的主要功能": each host
 * attends over the anchor block, the passing block and its local block; the
 * passing block is dropped afterwards).  Local query row r of q head i
 * (kv head h = map[i]) sees every anchor row, every passing row and local rows
 * 0..r of kv head h:
 *     O[r][i] = softmax(scale * q[r][i] . K^T) V,   lse[i][r] = ln(sum exp(...))
 *   q_local            bf16 [L][Hq][d]
 *   k_anchor, v_anchor bf16 [A][Hkv][d]  (may be NULL iff A == 0)
 *   k_pass, v_pass     bf16 [P][Hkv][d]  (may be NULL iff P == 0), P = p * l
 *   k_local, v_local   bf16 [L][Hkv][d]
 *   softmax_scale      finite, > 0 (commonly 1/sqrt(d))
 *   out                bf16 [L][Hq][d] (output, rounded to nearest even)
 *   lse                fp32 [Hq][L]    (output, natural log) or NULL
 * bf16 products, fp32 accumulation and fp32 online softmax.
 */
apb_status apb_block_attention(const apb_problem *problem, const void *q_local,
                               const void *k_anchor, const void *v_anchor,
                               const void *k_pass, const void *v_pass,
                               const void *k_local, const void *v_local,
                               float softmax_scale, void *out, float *lse, void *stream);

/*
 * Key segments of step 4, for computing it in parts.  The passing block is the
 * only input that depends on the exchange between hosts (explainer,
 * "APB 的主要功能": the compressed blocks are all-gathered into the passing block,
 * then each host attends over anchor, passing and local blocks), so a host can
 * attend over anchor + local while the exchange is in flight, attend over the
 * passing block once it has arrived, and merge the two partial results.
 */
#define APB_SEG_ANCHOR 1u
#define APB_SEG_PASSING 2u
#define APB_SEG_LOCAL 4u
#define APB_SEG_ALL 7u

/*
 * Step 4 restricted to the key segments in `segments` (a non-zero OR of
 * APB_SEG_*): local query row r sees the anchor rows if APB_SEG_ANCHOR is set,
 * the passing rows if APB_SEG_PASSING is set and local rows 0..r if
 * APB_SEG_LOCAL is set.  Arguments as for apb_block_attention; the key/value
 * pointers of segments left out are ignored and may be NULL.  A row that sees
 * no key at all (LOCAL left out and the selected segments empty) gets O = 0
 * and lse = -inf, the identity of apb_merge_attention.
 * apb_block_attention is this call with APB_SEG_ALL.
 */
apb_status apb_block_attention_segments(const apb_problem *problem, uint32_t segments, const void *q_local,
                                        const void *k_anchor, const void *v_anchor,
                                        const void *k_pass, const void *v_pass,
                                        const void *k_local, const void *v_local,
                                        float softmax_scale, void *out, float *lse, void *stream);

/*
 * Merge two partial attention results over disjoint key sets into the result
 * over their union: per q head i and local row r, with m = max(lse_a, lse_b),
 *     w_a = exp(lse_a - m),  w_b = exp(lse_b - m)
 *     out = (w_a * out_a + w_b * out_b) / (w_a + w_b),  lse = m + ln(w_a + w_b)
 * (softmax over a union of key sets; the same identity FlashAttention's
 * online softmax uses between key tiles).  Rows where both lse are -inf give
 * out = 0, lse = -inf.  Computed in fp32.
 *   out_a, out_b  bf16 [L][Hq][d]     lse_a, lse_b  fp32 [Hq][L] (required)
 *   out           bf16 [L][Hq][d] (output; may be out_a or out_b itself)
 *   lse           fp32 [Hq][L] (output; may be lse_a or lse_b itself) or NULL
 * Only n_q_heads, head_dim and local_len of `problem` are used, but the whole
 * problem must be valid.
 */
apb_status apb_merge_attention(const apb_problem *problem, const void *out_a, const float *lse_a,
                               const void *out_b, const float *lse_b, void *out, float *lse, void *stream);

/*
 * The steps on either side of step 4 in one layer on a host.
 *
 * Each host carries the anchor through the layer together with its local block
 * (explainer, "APB 的主要功能": the anchor block, holding the start of the
 * sequence, is prepended to every local block), so the anchor's own queries
 * attend causally over the anchor: anchor row r sees anchor rows 0..r.
 *   q_anchor            bf16 [A][Hq][d]
 *   k_anchor, v_anchor  bf16 [A][Hkv][d]
 *   out                 bf16 [A][Hq][d] (output)
 *   lse                 fp32 [Hq][A]    (output, natural log) or NULL
 * Requires A >= 1; uses the step-4 kernel.  Other arguments as apb_block_attention.
 */
apb_status apb_anchor_attention(const apb_problem *problem, const void *q_anchor, const void *k_anchor,
                                const void *v_anchor, float softmax_scale, void *out, float *lse, void *stream);

/*
 * Rotary position embedding, rotate-half pairing, on a token-major tensor (the
 * position encoding of the Llama models the pages evaluate on; q and k reach
 * the steps above already rotated).  Row r sits at position pos0 + r; for head
 * h and i < d/2, with theta_i = theta_base^(-2i/d) and a = (pos0 + r) * theta_i:
 *     out[r][h][i]       = x[r][h][i] cos(a) - x[r][h][i + d/2] sin(a)
 *     out[r][h][i + d/2] = x[r][h][i] sin(a) + x[r][h][i + d/2] cos(a)
 *   x, out   bf16 [rows][heads][d], d in {64, 128}; out may be x (in place)
 * theta_i is computed on the host in double precision, a is formed and reduced
 * modulo 2*pi in double precision on the device, the rotation is done in fp32
 * and rounded once to bf16 (nearest even).  Positions are capped so that the
 * double-precision angle stays within 2^31 * 2^-52 = 2^-21 rad of the exact one,
 * far below the bf16 rounding of the output.  rows >= 1, 1 <= heads <= 4096,
 * pos0 >= 0, pos0 + rows <= APB_MAX_ROPE_POSITION, theta_base > 1 and finite.
 */
apb_status apb_rope(const void *x, void *out, int32_t rows, int32_t heads, int32_t head_dim, int64_t pos0,
                    float theta_base, void *stream);

/*
 * QKV projection of `rows` hidden-state rows of a host (its local block, or
 * the anchor it carries), before step 1: with nn.Linear weights [out][in],
 *     q = x Wq^T,  k = x Wk^T,  v = x Wv^T
 *   x        bf16 [rows][hidden]
 *   wq       bf16 [Hq*d][hidden];   wk, wv  bf16 [Hkv*d][hidden]
 *   q        bf16 [rows][Hq][d];    k, v    bf16 [rows][Hkv][d]   (outputs)
 * Products of bf16 values accumulate in fp32; each output is rounded once to
 * bf16 (nearest even).  hidden: a multiple of 32, 32..1048576; 1 <= rows <=
 * APB_MAX_LOCAL_LEN.  Only n_q_heads, n_kv_heads and head_dim of `problem` are
 * used, but the whole problem must be valid.  One kernel launch computes q, k
 * and v.
 */
apb_status apb_qkv_projection(const apb_problem *problem, int32_t rows, int32_t hidden, const void *x,
                              const void *wq, const void *wk, const void *wv, void *q, void *k, void *v,
                              void *stream);

/* Host-only checks of a problem description; launches nothing. */
apb_status apb_validate_problem(const apb_problem *problem);

/* Static text for a status code. */
const char *apb_status_string(apb_status status);

/* Message describing the calling thread's most recent error ("" if none). */
const char *apb_last_error(void);

/* APB_ABI_VERSION of the loaded library. */
int apb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* APB_H */
