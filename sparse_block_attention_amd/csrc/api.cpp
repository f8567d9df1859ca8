// C-ABI entry points: check arguments on the host, then launch the HIP kernels
// on the caller's stream.  Nothing is allocated; no exception crosses the ABI.
#include <math.h>
#include <string.h>

#include "apb_host.h"
#include "apb_internal.h"

using apb_host::aligned16;
using apb_host::fail;

namespace {

apb_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return APB_OK;
  return fail(APB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

apb_status need_ptr(const void *p, const char *name) {
  if (p == nullptr) return fail(APB_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(APB_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return APB_OK;
}

#define APB_TRY(expr)              \
  do {                             \
    apb_status st_ = (expr);       \
    if (st_ != APB_OK) return st_; \
  } while (0)

apb_status score_kv(const apb_problem *pr, const apb_scorer *sc, const void *q, const void *k, const void *v,
                    float *scores, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (sc == nullptr) return fail(APB_ERR_INVALID_ARGUMENT, "scorer is NULL");
  if (sc->hidden < 16 || sc->hidden > 256 || sc->hidden % 16 != 0)
    return fail(APB_ERR_UNSUPPORTED, "scorer hidden = %d, supported: multiples of 16 in [16, 256]", sc->hidden);
  APB_TRY(need_ptr(sc->w1, "scorer.w1"));
  APB_TRY(need_ptr(sc->b1, "scorer.b1"));
  APB_TRY(need_ptr(sc->w2, "scorer.w2"));
  APB_TRY(need_ptr(sc->b2, "scorer.b2"));
  APB_TRY(need_ptr(q, "q_local"));
  APB_TRY(need_ptr(k, "k_local"));
  APB_TRY(need_ptr(v, "v_local"));
  APB_TRY(need_ptr(scores, "scores"));
  apb::ScoreArgs a;
  memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t *>(q);
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.w1 = static_cast<const uint16_t *>(sc->w1);
  a.b1 = sc->b1;
  a.w2 = sc->w2;
  a.b2 = sc->b2;
  a.scores = scores;
  a.L = pr->local_len;
  a.Hq = pr->n_q_heads;
  a.Hkv = pr->n_kv_heads;
  a.g = pr->n_q_heads / pr->n_kv_heads;
  a.d = pr->head_dim;
  a.hidden = sc->hidden;
  apb_host::slot_table(pr, a.qhead_of_slot);
  return hip_status(apb::launch_score_kv(a, static_cast<hipStream_t>(stream)), "apb_score_kv launch");
}

// Checks shared by both top-l entry points (the problem is already valid, l > 0).
apb_status check_topk_pointers(const float *scores, const void *k, const void *v, const int32_t *idx,
                               const void *kc, const void *vc) {
  APB_TRY(need_ptr(scores, "scores"));
  APB_TRY(need_ptr(k, "k_local"));
  APB_TRY(need_ptr(v, "v_local"));
  APB_TRY(need_ptr(idx, "idx"));
  APB_TRY(need_ptr(kc, "k_comp"));
  APB_TRY(need_ptr(vc, "v_comp"));
  return APB_OK;
}

apb_status launch_topk(const apb_problem *pr, const float *scores, const void *k, const void *v, int32_t *idx,
                       void *kc, void *vc, void *ws, void *stream) {
  apb::TopkArgs a;
  memset(&a, 0, sizeof a);
  a.scores = scores;
  a.k = static_cast<const uint16_t *>(k);
  a.v = static_cast<const uint16_t *>(v);
  a.idx = idx;
  a.kc = static_cast<uint16_t *>(kc);
  a.vc = static_cast<uint16_t *>(vc);
  a.L = pr->local_len;
  a.l = pr->pass_per_host;
  a.Hkv = pr->n_kv_heads;
  a.d = pr->head_dim;
  return hip_status(apb::launch_topk_gather(a, ws, static_cast<hipStream_t>(stream)), "apb_topk_gather launch");
}

apb_status topk_gather(const apb_problem *pr, const float *scores, const void *k, const void *v, int32_t *idx,
                       void *kc, void *vc, void *ws, size_t ws_bytes, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (pr->pass_per_host == 0) return APB_OK;
  APB_TRY(check_topk_pointers(scores, k, v, idx, kc, vc));
  const size_t need_bytes = apb::topk_workspace_bytes(pr->local_len, pr->n_kv_heads);
  if (ws_bytes < need_bytes)
    return fail(APB_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes = %zu, need %zu (apb_topk_workspace_size)", ws_bytes,
                need_bytes);
  APB_TRY(need_ptr(ws, "workspace"));
  return launch_topk(pr, scores, k, v, idx, kc, vc, ws, stream);
}

apb_status topk_gather_noalloc(const apb_problem *pr, const float *scores, const void *k, const void *v,
                               int32_t *idx, void *kc, void *vc, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (pr->pass_per_host == 0) return APB_OK;
  APB_TRY(check_topk_pointers(scores, k, v, idx, kc, vc));
  const size_t need_bytes = apb::topk_workspace_bytes(pr->local_len, pr->n_kv_heads);
  if (need_bytes > apb::kStaticTopkScratchBytes)
    return fail(APB_ERR_UNSUPPORTED,
                "apb_topk_gather_noalloc: this problem needs %zu bytes of workspace, the static workspace holds "
                "%zu (APB_NOALLOC_TOPK_WORKSPACE_BYTES); use apb_topk_gather with a caller workspace",
                need_bytes, apb::kStaticTopkScratchBytes);
  void *ws = nullptr;
  APB_TRY(hip_status(apb::static_topk_scratch(&ws), "apb_topk_gather_noalloc: static workspace address"));
  return launch_topk(pr, scores, k, v, idx, kc, vc, ws, stream);
}

size_t topk_workspace_size(const apb_problem *pr) {
  if (apb_host::check_problem(pr) != APB_OK) return 0;
  if (pr->pass_per_host == 0) return 0;
  return apb::topk_workspace_bytes(pr->local_len, pr->n_kv_heads);
}

apb_status build_passing(const apb_problem *pr, const void *const *kh, const void *const *vh, void *kp, void *vp,
                         void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  const int p = pr->host_index;
  const long long l = pr->pass_per_host;
  if (p == 0 || l == 0) return APB_OK;
  if (kh == nullptr || vh == nullptr) return fail(APB_ERR_INVALID_ARGUMENT, "host pointer arrays are NULL");
  APB_TRY(need_ptr(kp, "k_pass"));
  APB_TRY(need_ptr(vp, "v_pass"));
  for (int j = 0; j < p; ++j) {
    if (kh[j] == nullptr || !aligned16(kh[j]))
      return fail(APB_ERR_INVALID_ARGUMENT, "k_comp_hosts[%d] is NULL or not 16-byte aligned", j);
    if (vh[j] == nullptr || !aligned16(vh[j]))
      return fail(APB_ERR_INVALID_ARGUMENT, "v_comp_hosts[%d] is NULL or not 16-byte aligned", j);
  }
  const long long units = l * pr->n_kv_heads * pr->head_dim / 8;  // 16-byte units per block
  for (int j0 = 0; j0 < p; j0 += APB_MAX_PASS_HOSTS_PER_LAUNCH) {
    apb::PassArgs a;
    memset(&a, 0, sizeof a);
    const int n = (p - j0 < APB_MAX_PASS_HOSTS_PER_LAUNCH) ? p - j0 : APB_MAX_PASS_HOSTS_PER_LAUNCH;
    for (int j = 0; j < n; ++j) {
      a.ksrc[j] = static_cast<const uint16_t *>(kh[j0 + j]);
      a.vsrc[j] = static_cast<const uint16_t *>(vh[j0 + j]);
    }
    a.kdst = static_cast<uint16_t *>(kp) + (long long)j0 * units * 8;
    a.vdst = static_cast<uint16_t *>(vp) + (long long)j0 * units * 8;
    a.block_u16x8 = units;
    a.n_src = n;
    APB_TRY(hip_status(apb::launch_build_passing(a, static_cast<hipStream_t>(stream)), "apb_build_passing launch"));
  }
  return APB_OK;
}

apb_status block_attention(const apb_problem *pr, uint32_t segments, const void *q, const void *ka,
                           const void *va, const void *kp, const void *vp, const void *kl, const void *vl,
                           float scale, void *out, float *lse, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (segments == 0 || (segments & ~APB_SEG_ALL) != 0)
    return fail(APB_ERR_INVALID_ARGUMENT, "segments = 0x%x, need a non-zero OR of APB_SEG_*", (unsigned)segments);
  const bool use_a = (segments & APB_SEG_ANCHOR) != 0;
  const bool use_p = (segments & APB_SEG_PASSING) != 0;
  const bool use_l = (segments & APB_SEG_LOCAL) != 0;
  const long long A = use_a ? pr->anchor_len : 0;
  const long long P = use_p ? (long long)pr->host_index * pr->pass_per_host : 0;
  APB_TRY(need_ptr(q, "q_local"));
  APB_TRY(need_ptr(out, "out"));
  if (use_l) {
    APB_TRY(need_ptr(kl, "k_local"));
    APB_TRY(need_ptr(vl, "v_local"));
  }
  if (A > 0) {
    APB_TRY(need_ptr(ka, "k_anchor"));
    APB_TRY(need_ptr(va, "v_anchor"));
  }
  if (P > 0) {
    APB_TRY(need_ptr(kp, "k_pass"));
    APB_TRY(need_ptr(vp, "v_pass"));
  }
  if (lse != nullptr && !aligned16(lse)) return fail(APB_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(APB_ERR_INVALID_ARGUMENT, "softmax_scale = %g, need finite and > 0", (double)scale);
  apb::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t *>(q);
  a.ka = A > 0 ? static_cast<const uint16_t *>(ka) : nullptr;
  a.va = A > 0 ? static_cast<const uint16_t *>(va) : nullptr;
  a.kp = P > 0 ? static_cast<const uint16_t *>(kp) : nullptr;
  a.vp = P > 0 ? static_cast<const uint16_t *>(vp) : nullptr;
  a.kl = use_l ? static_cast<const uint16_t *>(kl) : nullptr;
  a.vl = use_l ? static_cast<const uint16_t *>(vl) : nullptr;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  a.L = pr->local_len;
  a.A = (int)A;
  a.P = (int)P;
  a.use_local = use_l ? 1 : 0;
  a.Hq = pr->n_q_heads;
  a.Hkv = pr->n_kv_heads;
  a.g = pr->n_q_heads / pr->n_kv_heads;
  a.scale_log2 = scale * 1.4426950408889634f;
  apb_host::slot_table(pr, a.qhead_of_slot);
  return hip_status(apb::launch_block_attention(a, pr->head_dim, static_cast<hipStream_t>(stream)),
                    "apb_block_attention launch");
}

apb_status anchor_attention(const apb_problem *pr, const void *q, const void *k, const void *v, float scale,
                            void *out, float *lse, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (pr->anchor_len < 1) return fail(APB_ERR_INVALID_ARGUMENT, "anchor attention needs anchor_len >= 1");
  // The anchor's own rows as a local block: causal, no anchor, no passing.
  apb_problem ap = *pr;
  ap.local_len = pr->anchor_len;
  ap.anchor_len = 0;
  ap.pass_per_host = 0;
  ap.host_index = 0;
  ap.n_hosts = 1;
  APB_TRY(apb_host::check_problem(&ap));
  return block_attention(&ap, APB_SEG_LOCAL, q, nullptr, nullptr, nullptr, nullptr, k, v, scale, out, lse, stream);
}

apb_status rope(const void *x, void *out, int32_t rows, int32_t heads, int32_t d, int64_t pos0, float base,
                void *stream) {
  APB_TRY(need_ptr(x, "x"));
  APB_TRY(need_ptr(out, "out"));
  if (rows < 1) return fail(APB_ERR_INVALID_ARGUMENT, "rows = %d, need >= 1", rows);
  if (heads < 1 || heads > 4096) return fail(APB_ERR_INVALID_ARGUMENT, "heads = %d, need 1..4096", heads);
  if (d != 64 && d != 128) return fail(APB_ERR_UNSUPPORTED, "head_dim = %d, supported: 64, 128", d);
  if (pos0 < 0 || pos0 + rows > APB_MAX_ROPE_POSITION)
    return fail(APB_ERR_INVALID_ARGUMENT, "pos0 = %lld, rows = %d: positions must lie in [0, 2^31)",
                (long long)pos0, rows);
  if (!(base > 1.f) || !isfinite(base))
    return fail(APB_ERR_INVALID_ARGUMENT, "theta_base = %g, need finite and > 1", (double)base);
  apb::RopeArgs a;
  memset(&a, 0, sizeof a);
  a.x = static_cast<const uint16_t *>(x);
  a.out = static_cast<uint16_t *>(out);
  a.pos0 = pos0;
  a.rows = rows;
  a.heads = heads;
  a.d = d;
  for (int i = 0; i < d / 2; ++i) a.theta[i] = pow((double)base, -2.0 * i / d);
  return hip_status(apb::launch_rope(a, static_cast<hipStream_t>(stream)), "apb_rope launch");
}

apb_status qkv_projection(const apb_problem *pr, int32_t rows, int32_t hidden, const void *x, const void *wq,
                          const void *wk, const void *wv, void *q, void *k, void *v, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  if (rows < 1 || rows > APB_MAX_LOCAL_LEN)
    return fail(APB_ERR_INVALID_ARGUMENT, "rows = %d, need 1..%d", rows, APB_MAX_LOCAL_LEN);
  if (hidden < 32 || hidden > (1 << 20) || hidden % 32 != 0)
    return fail(APB_ERR_UNSUPPORTED, "hidden = %d, supported: multiples of 32 in [32, 2^20]", hidden);
  const void *ins[4] = {x, wq, wk, wv};
  const char *in_names[4] = {"x", "wq", "wk", "wv"};
  for (int i = 0; i < 4; ++i) APB_TRY(need_ptr(ins[i], in_names[i]));
  APB_TRY(need_ptr(q, "q"));
  APB_TRY(need_ptr(k, "k"));
  APB_TRY(need_ptr(v, "v"));
  const int d = pr->head_dim;
  apb::ProjArgs a;
  memset(&a, 0, sizeof a);
  a.x = static_cast<const uint16_t *>(x);
  a.w[0] = static_cast<const uint16_t *>(wq);
  a.w[1] = static_cast<const uint16_t *>(wk);
  a.w[2] = static_cast<const uint16_t *>(wv);
  a.c[0] = static_cast<uint16_t *>(q);
  a.c[1] = static_cast<uint16_t *>(k);
  a.c[2] = static_cast<uint16_t *>(v);
  a.N[0] = pr->n_q_heads * d;
  a.N[1] = pr->n_kv_heads * d;
  a.N[2] = pr->n_kv_heads * d;
  a.M = rows;
  a.K = hidden;
  APB_TRY(hip_status(apb::launch_proj_gemm(a, static_cast<hipStream_t>(stream)), "apb_qkv_projection launch"));
  return APB_OK;
}

apb_status merge_attention(const apb_problem *pr, const void *oa, const float *la, const void *ob, const float *lb,
                           void *out, float *lse, void *stream) {
  APB_TRY(apb_host::check_problem(pr));
  APB_TRY(need_ptr(oa, "out_a"));
  APB_TRY(need_ptr(la, "lse_a"));
  APB_TRY(need_ptr(ob, "out_b"));
  APB_TRY(need_ptr(lb, "lse_b"));
  APB_TRY(need_ptr(out, "out"));
  if (lse != nullptr && !aligned16(lse)) return fail(APB_ERR_INVALID_ARGUMENT, "lse is not 16-byte aligned");
  apb::MergeArgs a;
  a.oa = static_cast<const uint16_t *>(oa);
  a.ob = static_cast<const uint16_t *>(ob);
  a.la = la;
  a.lb = lb;
  a.out = static_cast<uint16_t *>(out);
  a.lse = lse;
  a.L = pr->local_len;
  a.Hq = pr->n_q_heads;
  a.d = pr->head_dim;
  return hip_status(apb::launch_merge_attention(a, static_cast<hipStream_t>(stream)), "apb_merge_attention launch");
}

}  // namespace

#define APB_GUARD(call)                                                 \
  try {                                                                 \
    apb_host::clear_error();                                            \
    return call;                                                        \
  } catch (...) {                                                       \
    return fail(APB_ERR_INTERNAL, "unexpected C++ exception in %s", __func__); \
  }

extern "C" {

apb_status apb_score_kv(const apb_problem *problem, const apb_scorer *scorer, const void *q_local,
                        const void *k_local, const void *v_local, float *scores, void *stream) {
  APB_GUARD(score_kv(problem, scorer, q_local, k_local, v_local, scores, stream));
}

size_t apb_topk_workspace_size(const apb_problem *problem) {
  try {
    apb_host::clear_error();
    return topk_workspace_size(problem);
  } catch (...) {
    fail(APB_ERR_INTERNAL, "unexpected C++ exception in %s", __func__);
    return 0;
  }
}

apb_status apb_topk_gather(const apb_problem *problem, const float *scores, const void *k_local,
                           const void *v_local, int32_t *idx, void *k_comp, void *v_comp, void *workspace,
                           size_t workspace_bytes, void *stream) {
  APB_GUARD(topk_gather(problem, scores, k_local, v_local, idx, k_comp, v_comp, workspace, workspace_bytes,
                        stream));
}

apb_status apb_topk_gather_noalloc(const apb_problem *problem, const float *scores, const void *k_local,
                                   const void *v_local, int32_t *idx, void *k_comp, void *v_comp, void *stream) {
  APB_GUARD(topk_gather_noalloc(problem, scores, k_local, v_local, idx, k_comp, v_comp, stream));
}

apb_status apb_build_passing(const apb_problem *problem, const void *const *k_comp_hosts,
                             const void *const *v_comp_hosts, void *k_pass, void *v_pass, void *stream) {
  APB_GUARD(build_passing(problem, k_comp_hosts, v_comp_hosts, k_pass, v_pass, stream));
}

apb_status apb_block_attention(const apb_problem *problem, const void *q_local, const void *k_anchor,
                               const void *v_anchor, const void *k_pass, const void *v_pass, const void *k_local,
                               const void *v_local, float softmax_scale, void *out, float *lse, void *stream) {
  APB_GUARD(block_attention(problem, APB_SEG_ALL, q_local, k_anchor, v_anchor, k_pass, v_pass, k_local, v_local,
                            softmax_scale, out, lse, stream));
}

apb_status apb_block_attention_segments(const apb_problem *problem, uint32_t segments, const void *q_local,
                                        const void *k_anchor, const void *v_anchor, const void *k_pass,
                                        const void *v_pass, const void *k_local, const void *v_local,
                                        float softmax_scale, void *out, float *lse, void *stream) {
  APB_GUARD(block_attention(problem, segments, q_local, k_anchor, v_anchor, k_pass, v_pass, k_local, v_local,
                            softmax_scale, out, lse, stream));
}

apb_status apb_anchor_attention(const apb_problem *problem, const void *q_anchor, const void *k_anchor,
                                const void *v_anchor, float softmax_scale, void *out, float *lse, void *stream) {
  APB_GUARD(anchor_attention(problem, q_anchor, k_anchor, v_anchor, softmax_scale, out, lse, stream));
}

apb_status apb_rope(const void *x, void *out, int32_t rows, int32_t heads, int32_t head_dim, int64_t pos0,
                    float theta_base, void *stream) {
  APB_GUARD(rope(x, out, rows, heads, head_dim, pos0, theta_base, stream));
}

apb_status apb_qkv_projection(const apb_problem *problem, int32_t rows, int32_t hidden, const void *x,
                              const void *wq, const void *wk, const void *wv, void *q, void *k, void *v,
                              void *stream) {
  APB_GUARD(qkv_projection(problem, rows, hidden, x, wq, wk, wv, q, k, v, stream));
}

apb_status apb_merge_attention(const apb_problem *problem, const void *out_a, const float *lse_a, const void *out_b,
                               const float *lse_b, void *out, float *lse, void *stream) {
  APB_GUARD(merge_attention(problem, out_a, lse_a, out_b, lse_b, out, lse, stream));
}

}  // extern "C"
