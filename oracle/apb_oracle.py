"""CPU oracle for the APB per-host prefill path.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package entry's smoke check and the benchmark's CPU-baseline
leg may import or run this module.  The product path never does: it shares no
code with this file and fails if its HIP library is missing.

Plain, slow numpy in float64, one step per function, in the order the pages give:
  1. score each kv head's local tokens (stand-in for Locret's retaining heads),
  2. keep the l highest-scoring tokens per kv head and gather their K/V rows
     (the compressed context block),
  3. concatenate the compressed blocks of the preceding hosts (the passing block),
  4. attention of the local queries over [anchor | passing | local, causal],
     also over any subset of those key segments, and the merge of two partial
     results over disjoint key sets into the result over their union;
and, either side of step 4, the QKV projection and rotary position embedding of
q and k.

Sources (web pages on APB, "Accelerating Distributed Long-Context Inference by
Passing Compressed Context Blocks across GPUs"):
  * arXiv abstract (mlsanity.com/paper/2502.12085): multi-host approximate
    attention that passes essential KV pairs, run by a FlashAttention kernel
    adapted to APB.
  * juejin.cn explainer, section "APB 的主要功能": the input is split evenly over
    hosts and an anchor block holding the start of the sequence is prepended to
    each local block; each host compresses its KV cache with retaining heads;
    the compressed blocks are all-gathered and the passing block carries the
    important KV of the preceding hosts; attention combines anchor, passing and
    local blocks, and the passing block is dropped afterwards.
  * same page, section "APB 的技术原理": smaller anchor (1/4 or 1/8 of a block);
    passing block built from the important KV pairs of earlier devices; the
    query is embedded at the start of the anchor so compression is query-aware.

Readings where the pages are silent (each also listed in the design doc):
  scale 1/sqrt(d); anchor and passing keys fully visible, local keys causal;
  the scorer is a per-kv-head 2-layer ReLU MLP on [q of the group's heads
  (ascending q-head order); k; v]; scores are rounded to fp32 before selection;
  order is larger fp32 value first, -0 equal to +0, NaN below -inf, ties to the
  lower token index; selected indices are stored ascending; the passing block is
  host-major (row j*l + s); selection runs over the whole local block.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _head_map(n_q_heads: int, n_kv_heads: int, kv_head_of_q=None) -> np.ndarray:
    if kv_head_of_q is None:
        g = n_q_heads // n_kv_heads
        return np.array([i // g for i in range(n_q_heads)], dtype=np.int64)
    m = np.asarray(kv_head_of_q, dtype=np.int64)
    if m.shape != (n_q_heads,):
        raise ValueError("head map must have one entry per q head")
    return m


def group_of(kv_head: int, head_map: np.ndarray) -> list:
    """q heads attached to one kv head, in ascending q-head order."""
    return [i for i in range(len(head_map)) if head_map[i] == kv_head]


# ---------------------------------------------------------------------------
# Step 1: per-kv-head importance score (retaining-head stand-in).
# explainer, section "APB 的主要功能", bullet on compressing the KV cache with
# retaining heads; section "APB 的技术原理", bullet on query-aware compression.
# ---------------------------------------------------------------------------
def score_kv(q, k, v, w1, b1, w2, b2, kv_head_of_q=None) -> np.ndarray:
    """fp32 [Hkv, L] scores s[h,t] = w2[h] . relu(W1[h] x + b1[h]) + b2[h].

    x = [q[t, G_h[0]]; ...; q[t, G_h[g-1]]; k[t, h]; v[t, h]] with G_h the q
    heads mapped to kv head h in ascending order.  Computed in float64 and
    rounded once to float32.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    w1, b1, w2, b2 = _f64(w1), _f64(b1), _f64(w2), _f64(b2)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    hm = _head_map(Hq, Hkv, kv_head_of_q)
    out = np.empty((Hkv, L), dtype=np.float32)
    for h in range(Hkv):
        parts = [q[:, i, :] for i in group_of(h, hm)] + [k[:, h, :], v[:, h, :]]
        x = np.concatenate(parts, axis=1)                 # [L, (g+2)d]
        z = x @ w1[h].T + b1[h]                           # [L, Hs]
        s = np.maximum(z, 0.0) @ w2[h] + b2[h]            # [L]
        out[h] = s.astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# Step 2: keep the l most important tokens of each kv head.
# explainer, "APB 的主要功能" (compress the KV cache, keep the important KV
# units) and "APB 的技术原理" (passing block of important KV pairs).
# ---------------------------------------------------------------------------
def topl_one(scores_row, l: int) -> np.ndarray:
    """Ascending local indices of the l best entries of one fp32 score row.

    Order: larger value first; -0 == +0; NaN after every number (even -inf);
    equal values go to the lower index.
    """
    s = np.asarray(scores_row, dtype=np.float32)
    n = s.shape[0]
    if not 0 <= l <= n:
        raise ValueError("need 0 <= l <= number of tokens")
    nan = np.isnan(s)
    val = np.where(nan, np.float32(0), s).astype(np.float64)
    idx = np.arange(n)
    # np.lexsort sorts by the last key first: NaN flag, then -value, then index.
    order = np.lexsort((idx, -val, nan.astype(np.int8)))
    return np.sort(order[:l]).astype(np.int32)


def topl(scores, l: int) -> np.ndarray:
    """int32 [Hkv, l]: per-kv-head selection (see topl_one)."""
    scores = np.asarray(scores, dtype=np.float32)
    return np.stack([topl_one(scores[h], l) for h in range(scores.shape[0])]) \
        if scores.shape[0] else np.zeros((0, l), np.int32)


# ---------------------------------------------------------------------------
# Step 2b: gather the selected rows into the compressed context block.
# explainer, "APB 的主要功能", bullet on the communication mechanism.
# ---------------------------------------------------------------------------
def gather(k, v, idx):
    """(k_comp, v_comp) [l, Hkv, d] with k_comp[s, h] = k[idx[h, s], h]."""
    k, v = np.asarray(k), np.asarray(v)
    Hkv, l = idx.shape
    kc = np.empty((l, Hkv, k.shape[2]), dtype=k.dtype)
    vc = np.empty((l, Hkv, v.shape[2]), dtype=v.dtype)
    for h in range(Hkv):
        kc[:, h, :] = k[idx[h], h, :]
        vc[:, h, :] = v[idx[h], h, :]
    return kc, vc


# ---------------------------------------------------------------------------
# Step 3: passing block = compressed blocks of the preceding hosts, in host order.
# explainer, "APB 的主要功能" (passing block of the preceding hosts' important
# KV) and "APB 的技术原理" (each block compressed and sent to later GPUs).
# ---------------------------------------------------------------------------
def build_passing(k_comps, v_comps):
    """(k_pass, v_pass) [p*l, Hkv, d]: row j*l + s holds slot s of host j (j < p)."""
    if len(k_comps) == 0:
        return None, None
    return np.concatenate(list(k_comps), axis=0), np.concatenate(list(v_comps), axis=0)


# ---------------------------------------------------------------------------
# Step 4: attention of the local queries over anchor, passing and local keys.
# explainer, "APB 的主要功能", bullet on computation (anchor + passing + local).
# ---------------------------------------------------------------------------
SEGMENTS_ALL = ("anchor", "passing", "local")


def block_attention(q, k_anchor, v_anchor, k_pass, v_pass, k_local, v_local,
                    scale=None, kv_head_of_q=None, rows=None, heads=None,
                    chunk: int = 256, segments=SEGMENTS_ALL):
    """Masked softmax attention in float64.

    Local query row r of q head i (kv head h = map[i]) sees every anchor row,
    every passing row and local rows 0..r (juejin.cn APB explainer, section
    "APB 的主要功能", computation bullet).  `segments` names the key segments
    attended (default all three); the arrays of segments left out are ignored.
    Returns (O [R, nH, d], lse [nH, R]) for the requested rows (default all) and
    q heads (default all); lse is the natural log of the softmax denominator
    including its max shift.  A row that sees no key gets O = 0, lse = -inf.
    """
    q = np.asarray(q)
    L, Hq, d = q.shape
    unknown = set(segments) - set(SEGMENTS_ALL)
    if unknown or not segments:
        raise ValueError(f"segments must be a non-empty subset of {SEGMENTS_ALL}")
    use_l = "local" in segments
    Hkv = (k_local if k_local is not None else (k_anchor if k_anchor is not None else k_pass)).shape[1]
    hm = _head_map(Hq, Hkv, kv_head_of_q)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)

    def seg(x, name):
        return _f64(x) if (x is not None and name in segments) else np.zeros((0, Hkv, d))

    ka, va = seg(k_anchor, "anchor"), seg(v_anchor, "anchor")
    kp, vp = seg(k_pass, "passing"), seg(v_pass, "passing")
    kl, vl = seg(k_local, "local"), seg(v_local, "local")
    n_pre = ka.shape[0] + kp.shape[0]
    out = np.empty((len(rows), len(heads), d), dtype=np.float64)
    lse = np.empty((len(heads), len(rows)), dtype=np.float64)
    for hi, i in enumerate(heads):
        h = hm[i]
        K = np.concatenate([ka[:, h], kp[:, h], kl[:, h]], axis=0)
        V = np.concatenate([va[:, h], vp[:, h], vl[:, h]], axis=0)
        for c0 in range(0, len(rows), chunk):
            rr = rows[c0:c0 + chunk]
            n_keys = n_pre + (int(rr.max()) + 1 if use_l else 0)
            if n_keys == 0:  # nothing visible to any of these rows
                out[c0:c0 + len(rr), hi, :] = 0.0
                lse[hi, c0:c0 + len(rr)] = -np.inf
                continue
            logits = scale * (_f64(q[rr, i, :]) @ K[:n_keys].T)      # [R, n_keys]
            local_col = np.arange(n_keys) - n_pre                      # local index or < 0
            visible = local_col[None, :] <= rr[:, None]
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            den = e.sum(axis=1, keepdims=True)
            out[c0:c0 + len(rr), hi, :] = (e @ V[:n_keys]) / den
            lse[hi, c0:c0 + len(rr)] = (m + np.log(den))[:, 0]
    return out, lse


def merge_attention(o_a, lse_a, o_b, lse_b):
    """Softmax over the union of two disjoint key sets from its two parts, float64.

    With partial results (o_x [R, nH, d], lse_x [nH, R]) over key sets X_a and
    X_b: the union's denominator is exp(lse_a) + exp(lse_b), and its output is
    the denominator-weighted mean of o_a and o_b.  Written with the max shift
    m = max(lse_a, lse_b) so nothing overflows; rows where both sides are empty
    (lse = -inf) give O = 0 and lse = -inf.
    """
    o_a, o_b = _f64(o_a), _f64(o_b)
    lse_a, lse_b = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w_a = np.exp(lse_a - m_safe)                 # exp(-inf) = 0 for an empty side
    w_b = np.exp(lse_b - m_safe)
    den = w_a + w_b
    nonempty = den > 0
    den_safe = np.where(nonempty, den, 1.0)
    c_a = (w_a / den_safe).T[:, :, None]          # [R, nH, 1]
    c_b = (w_b / den_safe).T[:, :, None]
    out = np.where(nonempty.T[:, :, None], c_a * o_a + c_b * o_b, 0.0)
    lse = np.where(nonempty, m_safe + np.log(den_safe), -np.inf)
    return out, lse


# ---------------------------------------------------------------------------
# Either side of step 4 (one layer on a host): the anchor's own causal
# attention is block_attention with the anchor as the local block and no other
# segment.  Rotary position embedding of q and k, rotate-half pairing (the
# position encoding of the Llama models the pages evaluate on).
# ---------------------------------------------------------------------------
def qkv_projection(x, wq, wk, wv, n_q_heads: int, n_kv_heads: int):
    """float64 (q [rows, Hq, d], k, v [rows, Hkv, d]) = x W^T for nn.Linear weights [out][in]."""
    x = _f64(x)
    rows = x.shape[0]
    q = (x @ _f64(wq).T).reshape(rows, n_q_heads, -1)
    k = (x @ _f64(wk).T).reshape(rows, n_kv_heads, -1)
    v = (x @ _f64(wv).T).reshape(rows, n_kv_heads, -1)
    return q, k, v


def rope(x, pos0: int, theta_base: float):
    """float64 [rows, heads, d]: row r at position pos0 + r; pair (i, i + d/2)
    rotated by the angle (pos0 + r) * theta_base^(-2i/d)."""
    x = _f64(x)
    rows, _, d = x.shape
    half = d // 2
    theta = float(theta_base) ** (-2.0 * np.arange(half) / d)
    ang = (pos0 + np.arange(rows, dtype=np.float64))[:, None] * theta[None, :]   # [rows, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x0, x1 = x[..., :half], x[..., half:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def compress_host(q, k, v, weights, l: int, kv_head_of_q=None):
    """Steps 1-2 for one host: (scores fp32 [Hkv,L], idx [Hkv,l], k_comp, v_comp)."""
    s = score_kv(q, k, v, weights["w1"], weights["b1"], weights["w2"], weights["b2"],
                 kv_head_of_q)
    idx = topl(s, l)
    kc, vc = gather(k, v, idx)
    return s, idx, kc, vc
