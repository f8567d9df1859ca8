"""Benchmark of the APB per-host prefill path on one MI355X.

One step = one host's share of one layer: score (apb_score_kv), top-l + gather
(apb_topk_gather), passing block (apb_build_passing) and attention
(apb_block_attention), on synthetic inputs already resident in HBM.  The
compressed blocks of the earlier hosts are produced before timing, in place of
the all-gather between hosts.  The host's own compression feeds later hosts,
not its own attention, so it runs on a second stream beside the passing build
and the attention (--serial puts everything on one stream).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b]

Prints one JSON line.  `value` is prefill tokens/s of the host block (L / step
time); `roofline` covers the attention kernel (HIP events around its launches);
`cpu_baseline` is the CPU oracle timed on a bounded sample of the same workload.

Extra objects (skipped with --no-extras):
  * `stages`: each step of the path alone on one stream (median and min of 20
    HIP-event timings, each behind a short spin kernel so that host overhead
    stays outside the events), warm and with the Infinity Cache evicted before
    every rep (by a 512 MB read; `cold_dirty` by a 512 MB write), with its
    algorithmic bytes (or FLOPs) and fraction of the HBM (or bf16 MFMA) peak,
    and scoring + top-l + gather combined; `sclk_mhz_after` is the shader
    clock level the amdgpu driver reports right after;
  * `split_phase`: anchor + local, then passing, then the merge of the two
    partial results (what lets the exchange between hosts overlap compute);
  * `modes`: the per-host attention of the two baselines the pages compare APB
    with, at the same layer shape: Star Attention (anchor = the whole first
    block, no passing block) and full causal FlashAttention-style attention of
    the last host (every earlier token visible, no anchor);
  * `layer_sides`: the QKV projection of the host block, rotary embedding of
    its q and k, and the anchor's own causal attention (steps either side of
    the attention step);
  * `workloads`: the other layer shapes (tiny, Qwen-2.5-14B, Yi-34B-200K,
    Llama-3-8B-1M), each step alone on seeded on-device inputs: attention
    (mean, median, min, TFLOP/s, fraction of peak) and the a1, a2+a3 and a5
    stages (warm and cold medians, fraction of HBM peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + prefill tokens/s per host block; % bf16 MFMA peak"
# MI355X dense bf16 MFMA peak: 256 CUs x 2.4 GHz x 4096 FLOP/CU/clock (the published 2.5 PFLOP/s).
PEAK_BF16_TFLOPS = 2516.6
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_attention_llama8b_traffic.json")
ATTN_SRC = os.path.join(ROOT, "sparse_block_attention_amd", "csrc", "block_attention.hip")

DESCRIPTIONS = {
    "llama8b": "Llama-3.1-8B-shaped layer, last of 8 hosts at 128K (L=16384, A=2048, P=7x1024)",
    "qwen14b": "Qwen-2.5-14B-shaped layer, last of 8 hosts at 128K (L=16384, A=4096, P=7x2048)",
    "yi34b": "Yi-34B-200K-shaped layer, last of 8 hosts at 200K (L=25600, A=3200, P=7x1600)",
    "llama1m": "Llama-3-8B-1M-shaped layer, last of 8 hosts at 1M (L=131072, A=16384, P=7x4096)",
    "tiny": "tiny: 1024 tokens over 4 hosts of 256, anchor 64, l=32",
}


def attention_flops(w) -> float:
    """Algorithmic FLOPs of the attention: QK^T and PV over the visible pairs only."""
    L, A, P = w.local_len, w.anchor_len, w.pass_len
    pairs = L * A + L * P + L * (L + 1) // 2
    return 4.0 * w.head_dim * w.n_q_heads * pairs


def attention_bytes(w) -> float:
    """Algorithmic HBM bytes of one attention launch: q, anchor/passing/local K and V read once,
    O and LSE written once."""
    d, Hq, Hkv = w.head_dim, w.n_q_heads, w.n_kv_heads
    L, A, P = w.local_len, w.anchor_len, w.pass_len
    return 2.0 * L * Hq * d * 2 + 2.0 * (A + P + L) * Hkv * d * 2 + 4.0 * Hq * L


def stage_bytes(w) -> dict:
    """Algorithmic HBM bytes of the compression steps and the passing build of one host."""
    L, Hq, Hkv, d, l = w.local_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.pass_per_host
    return {
        # q, k, v of the block read; fp32 scores written (the scorer weights stay in L2
        # and are not counted: scorer_weight_bytes)
        "a1_score": L * (Hq + 2 * Hkv) * d * 2 + Hkv * L * 4,
        # scores read; l rows of K and V per kv head read and written; indices written
        "a2a3_topl_gather": Hkv * L * 4 + 2 * 2 * l * Hkv * d * 2 + Hkv * l * 4,
        # the earlier hosts' compressed blocks of K and V read and written once
        "a5_passing": 2 * 2 * w.pass_len * Hkv * d * 2,
    }


def scorer_weight_bytes(w) -> int:
    """W1 (bf16), b1, w2 and b2 (fp32) of all kv heads: read by the scorer, L2-resident."""
    g = w.n_q_heads // w.n_kv_heads
    return w.n_kv_heads * w.hidden * (g + 2) * w.head_dim * 2 + w.n_kv_heads * (2 * w.hidden + 1) * 4


def _src_hash(path):
    """sha256 of a kernel source and the extra compiler options it is built with, so a
    record taken on one build is not applied to another."""
    from sparse_block_attention_amd import build as build_mod
    with open(path, "rb") as f:
        data = f.read()
    flags = " ".join(build_mod.EXTRA_FLAGS.get(os.path.basename(path), []))
    return hashlib.sha256(data + flags.encode()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, or None when
    absent, for another workload, or taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_sha256") != _src_hash(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


def _median_ms(fn, reps: int, warm: int) -> float:
    """Median of `reps` HIP-event timings of fn() on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def _stage_times(fn, reps: int, warm: int, evict=None):
    """Median and min (ms) of `reps` HIP-event timings of fn().  Before every rep a
    spin kernel that touches no memory holds the GPU for ~0.2 ms, so the host has
    queued fn()'s kernels before the start event is reached: the events then bracket
    GPU time only, not the host-side argument marshalling of a short kernel.  With
    `evict`, it runs before the spin (cold caches)."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        if evict is not None:
            evict()
        torch.cuda._sleep(400_000)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return float(np.median(t)), float(np.min(t))


def stages(B, w, pr, sc, host, ka, va, kcs, vcs, buf, reps=20, warm=5):
    """Each step of the path alone on one stream: score (a1), top-l + gather (a2+a3),
    passing build (a5) and attention (a6).  Warm: inputs as the previous rep left the
    caches.  Cold: a 512 MB buffer is read before every rep, outside the timed region,
    which evicts the 256 MB Infinity Cache and leaves it clean.  Cold dirty: the 512 MB
    buffer is written instead; the step then also pays for writing back the dirty lines."""
    import torch
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    scratch_i = scratch.view(torch.int32)
    total = torch.zeros((), dtype=torch.int64, device="cuda")
    fill = [0]

    def evict():
        # reading 512 MB leaves the Infinity Cache full of clean lines
        torch.sum(scratch_i, dim=0, out=total)

    def evict_dirty():
        # writing 512 MB leaves it full of dirty lines, whose write-back then
        # competes with the step's own reads
        fill[0] = (fill[0] + 1) & 0xFF
        scratch.fill_(fill[0])

    byt = stage_bytes(w)
    fns = {
        "a1_score": lambda: B.apb_score_kv(pr, sc, host.q, host.k, host.v, scores=buf.scores),
        "a2a3_topl_gather": lambda: B.apb_topk_gather(pr, buf.scores, host.k, host.v, idx=buf.idx,
                                                      k_comp=buf.k_comp, v_comp=buf.v_comp,
                                                      workspace=buf.topk_workspace),
    }
    if pr.pass_len:
        fns["a5_passing"] = lambda: B.apb_build_passing(pr, kcs, vcs, k_pass=buf.k_pass, v_pass=buf.v_pass)
    fns["a6_attention"] = lambda: B.apb_block_attention(pr, host.q, ka, va, buf.k_pass, buf.v_pass, host.k,
                                                        host.v, out=buf.out, lse=buf.lse)
    res = {}
    for name, fn in fns.items():
        med, mn = _stage_times(fn, reps, warm)
        r = {"us_median": med * 1e3, "us_min": mn * 1e3}
        if name in byt:
            cmed, cmn = _stage_times(fn, reps, warm, evict=evict)
            dmed, _ = _stage_times(fn, reps, warm, evict=evict_dirty)
            r.update({"cold_us_median": cmed * 1e3, "cold_us_min": cmn * 1e3, "cold_dirty_us_median": dmed * 1e3,
                      "bytes": byt[name], "gbs": byt[name] / (med * 1e-3) / 1e9,
                      "cold_gbs": byt[name] / (cmed * 1e-3) / 1e9})
            r["frac_hbm_peak"] = r["gbs"] / PEAK_HBM_GBS
            r["cold_frac_hbm_peak"] = r["cold_gbs"] / PEAK_HBM_GBS
        else:
            fl = attention_flops(w)
            r.update({"tflops": fl / (med * 1e-3) / 1e12, "frac_bf16_peak": fl / (med * 1e-3) / 1e12
                      / PEAK_BF16_TFLOPS})
        res[name] = r
    # scoring + top-l + gather together: their bytes over their summed time
    for tag in ("", "cold_", "cold_dirty_"):
        t = res["a1_score"][tag + "us_median"] + res["a2a3_topl_gather"][tag + "us_median"]
        b = byt["a1_score"] + byt["a2a3_topl_gather"]
        res[(tag or "warm_") + "a1_a3"] = {"us_median": t, "gbs": b / (t * 1e-6) / 1e9,
                              "frac_hbm_peak": b / (t * 1e-6) / 1e9 / PEAK_HBM_GBS}
    del scratch
    return res


def sclk_mhz():
    """Current shader clock level (MHz) from the amdgpu sysfs table of the first GPU that
    has one (the level in use is marked '*'), or None.  Read from sysfs, not rocm-smi, so
    that no child program starts."""
    import glob
    import re
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                        if m:
                            return int(m.group(1))
        except OSError:
            continue
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def split_phase(B, pr, host, ka, va, kp, vp, attn_ms, reps=10, warm=3):
    """Attention in two phases plus the merge, each timed alone (medians)."""
    import torch
    L, Hq, d = pr.local_len, pr.n_q_heads, pr.head_dim
    o1 = torch.empty((L, Hq, d), dtype=torch.bfloat16, device="cuda")
    o2, om = torch.empty_like(o1), torch.empty_like(o1)
    l1 = torch.empty((Hq, L), dtype=torch.float32, device="cuda")
    l2, lm = torch.empty_like(l1), torch.empty_like(l1)
    seg1 = B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL
    ph1 = _median_ms(lambda: B.apb_block_attention_segments(pr, seg1, host.q, ka, va, kp, vp, host.k, host.v,
                                                            out=o1, lse=l1), reps, warm)
    ph2 = _median_ms(lambda: B.apb_block_attention_segments(pr, B.APB_SEG_PASSING, host.q, ka, va, kp, vp,
                                                            host.k, host.v, out=o2, lse=l2), reps, warm)
    mg = _median_ms(lambda: B.apb_merge_attention(pr, o1, l1, o2, l2, out=om, lse=lm), reps, warm)
    merge_bytes = 3.0 * L * Hq * d * 2 + 3.0 * Hq * L * 4
    return {"ms_anchor_local": ph1, "ms_passing": ph2, "ms_merge": mg, "ms_total": ph1 + ph2 + mg,
            "ms_one_pass": attn_ms, "overhead_vs_one_pass": (ph1 + ph2 + mg) / attn_ms - 1.0,
            "merge_gbs": merge_bytes / (mg * 1e-3) / 1e9, "merge_frac_hbm_peak":
            merge_bytes / (mg * 1e-3) / 1e9 / PEAK_HBM_GBS}


def baseline_modes(B, w, host, prior_kv, attn_ms, reps=5, warm=2):
    """Per-host attention of Star Attention and of full causal attention, same kernel and shape."""
    import torch
    L, Hq, Hkv, d, p = w.local_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.host
    out = torch.empty((L, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, L), dtype=torch.float32, device="cuda")
    res = {}
    # Star Attention: the anchor is the whole first block; no passing block.
    k0, v0 = prior_kv[0]
    pr = B.Problem(Hq, Hkv, d, L, L, 0, p, w.n_hosts, None)
    ms = _median_ms(lambda: B.apb_block_attention(pr, host.q, k0, v0, None, None, host.k, host.v,
                                                  out=out, lse=lse), reps, warm)
    pairs = L * L + L * (L + 1) // 2
    res["star"] = {"anchor_len": L, "pass_len": 0, "ms": ms, "pairs_per_head": pairs}
    # Full causal attention of the last host: every earlier token visible, as one passing block.
    kf = torch.cat([kv[0] for kv in prior_kv])
    vf = torch.cat([kv[1] for kv in prior_kv])
    pr = B.Problem(Hq, Hkv, d, L, 0, L, p, w.n_hosts, None)
    ms = _median_ms(lambda: B.apb_block_attention(pr, host.q, None, None, kf, vf, host.k, host.v,
                                                  out=out, lse=lse), reps, warm)
    pairs = L * p * L + L * (L + 1) // 2
    res["full_causal"] = {"anchor_len": 0, "pass_len": p * L, "ms": ms, "pairs_per_head": pairs}
    del kf, vf
    apb_pairs = L * w.anchor_len + L * w.pass_len + L * (L + 1) // 2
    for m in res.values():
        fl = 4.0 * d * Hq * m["pairs_per_head"]
        m["tflops"] = fl / (m["ms"] * 1e-3) / 1e12
        m["frac_bf16_peak"] = m["tflops"] / PEAK_BF16_TFLOPS
        m["pairs_vs_apb"] = m["pairs_per_head"] / apb_pairs
        m["apb_attention_speedup"] = m["ms"] / attn_ms
    return res


def layer_sides(B, w, host, ka, va, reps=10, warm=3):
    """The steps either side of the attention step, timed alone (medians): rotary
    embedding of the host's q and k, and the anchor's own causal attention."""
    import torch
    L, A, Hq, Hkv, d = w.local_len, w.anchor_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    qo, ko = torch.empty_like(host.q), torch.empty_like(host.k)
    pos0 = w.host * L       # sequence position of the host block's first token
    ms_q = _median_ms(lambda: B.apb_rope(host.q, pos0, 500000.0, out=qo), reps, warm)
    ms_k = _median_ms(lambda: B.apb_rope(host.k, pos0, 500000.0, out=ko), reps, warm)
    rope_bytes = 2.0 * (L * Hq * d + L * Hkv * d) * 2
    res = {"rope_ms": ms_q + ms_k, "rope_gbs": rope_bytes / ((ms_q + ms_k) * 1e-3) / 1e9}
    res["rope_frac_hbm_peak"] = res["rope_gbs"] / PEAK_HBM_GBS
    # QKV projection of the host block from hidden states of width Hq*d (the
    # Llama layout: hidden = Hq * d), synthetic weights
    from sparse_block_attention_amd import synth
    from sparse_block_attention_amd.tensors import to_device_bf16
    hidden = Hq * d
    xs = torch.randn((L, hidden), dtype=torch.float32, device="cuda").to(torch.bfloat16)
    wts = [to_device_bf16(synth.random_bf16((n * d, hidden), 40 + i, sigma=hidden ** -0.5))
           for i, n in enumerate((Hq, Hkv, Hkv))]
    prp = B.Problem(Hq, Hkv, d, L, A, w.pass_per_host, w.host, w.n_hosts, None)
    qo2, ko2, vo2 = torch.empty_like(host.q), torch.empty_like(host.k), torch.empty_like(host.v)
    ms = _median_ms(lambda: B.apb_qkv_projection(prp, xs, *wts, q=qo2, k=ko2, v=vo2), reps, warm)
    fl = 2.0 * L * hidden * (Hq + 2 * Hkv) * d
    res.update({"qkv_projection_ms": ms, "qkv_projection_tflops": fl / (ms * 1e-3) / 1e12,
                "qkv_projection_frac_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
    del xs, wts, qo2, ko2, vo2
    if A:
        pr = B.Problem(Hq, Hkv, d, L, A, w.pass_per_host, w.host, w.n_hosts, None)
        qa = host.q[:A].contiguous()          # stand-in anchor queries of the anchor's shape
        out = torch.empty((A, Hq, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((Hq, A), dtype=torch.float32, device="cuda")
        ms = _median_ms(lambda: B.apb_anchor_attention(pr, qa, ka, va, out=out, lse=lse), reps, warm)
        fl = 4.0 * d * Hq * (A * (A + 1) // 2)
        res.update({"anchor_attention_ms": ms, "anchor_attention_tflops": fl / (ms * 1e-3) / 1e12})
    return res


def _tiny_step_single_thread():
    """Seconds for the whole tiny host step (scoring, top-l, gather, passing build and
    attention of every row) in the CPU oracle on one BLAS thread, or None without
    threadpoolctl."""
    from oracle import apb_oracle as orc
    from sparse_block_attention_amd import synth
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is optional
        return None
    wt = synth.WORKLOADS["tiny"]
    q, k, v = synth.host_block(wt, wt.host)
    wts = synth.scorer_weights(wt)
    ka, va = synth.anchor_kv(wt)
    comps = [(synth.random_bf16((wt.pass_per_host, wt.n_kv_heads, wt.head_dim), 92, stream=j),
              synth.random_bf16((wt.pass_per_host, wt.n_kv_heads, wt.head_dim), 93, stream=j))
             for j in range(wt.host)]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        s = orc.score_kv(q, k, v, wts["w1"], wts["b1"], wts["w2"], wts["b2"])
        orc.gather(k, v, orc.topl(s, wt.pass_per_host))
        kp, vp = orc.build_passing([c[0] for c in comps], [c[1] for c in comps])
        orc.block_attention(q, ka, va, kp, vp, k, v)
        t1 = time.perf_counter()
    return round(t1 - t0, 4)


def cpu_baseline(w, blocks, weights, anchor, n_rows=4096):
    """Time the CPU oracle on a bounded sample of one host step; scale to tokens/s."""
    from oracle import apb_oracle as orc
    from sparse_block_attention_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()
                     if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    q, k, v = blocks
    L = w.local_len
    t0 = time.perf_counter()
    s = orc.score_kv(q, k, v, weights["w1"], weights["b1"], weights["w2"], weights["b2"])
    t1 = time.perf_counter()
    idx = orc.topl(s, w.pass_per_host)
    orc.gather(k, v, idx)
    t2 = time.perf_counter()
    comps = [(synth.random_bf16((w.pass_per_host, w.n_kv_heads, w.head_dim), 90, stream=j),
              synth.random_bf16((w.pass_per_host, w.n_kv_heads, w.head_dim), 91, stream=j))
             for j in range(w.host)]
    t2b = time.perf_counter()
    kp, vp = orc.build_passing([c[0] for c in comps], [c[1] for c in comps])
    t3 = time.perf_counter()
    rows = np.linspace(0, L - 1, n_rows).round().astype(np.int64)
    orc.block_attention(q, anchor[0], anchor[1], kp, vp, k, v, rows=rows)
    t4 = time.perf_counter()
    pre = w.anchor_len + w.pass_len
    all_pairs = L * pre + L * (L + 1) // 2
    sample_pairs = int((pre + rows + 1).sum())
    t_attn = (t4 - t3) * all_pairs / sample_pairs
    t_total = (t1 - t0) + (t2 - t1) + (t3 - t2b) + t_attn
    return {
        "value": L / t_total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "tiny_step_single_thread_s": _tiny_step_single_thread(),
        "sample": (f"scoring, top-l and gather over the whole {L}-token block; passing build of "
                   f"{w.host} blocks; attention for {n_rows} evenly spaced query rows x "
                   f"{w.n_q_heads} heads ({sample_pairs} of {all_pairs} visible pairs per head, "
                   f"scaled by the pair count); float64 numpy"),
        "seconds_measured": round(t4 - t0, 2), "seconds_extrapolated": round(t_total, 2),
        "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
    }


def _attention_stats(ms_list, flops):
    ms = np.asarray(ms_list, dtype=np.float64)
    mean, med, mn = float(ms.mean()), float(np.median(ms)), float(ms.min())
    return {"ms": mean, "ms_median": med, "ms_min": mn, "launches": int(ms.size),
            "tflops": flops / (mean * 1e-3) / 1e12, "frac_bf16_peak": flops / (mean * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "tflop_per_launch": flops / 1e12}


def other_workloads(B, names, reps=10, warm=3):
    """Each step of the path alone at the other layer shapes, on seeded on-device inputs
    (torch generator, N(0, 0.5^2) rounded to bf16; random compressed blocks of the earlier
    hosts; random scorer weights): attention (HIP events around every launch, mean, median
    and min) and the a1, a2+a3 and a5 stages (warm and cold medians).  Parity at these
    shapes is covered by the GPU tests; this measures throughput."""
    import torch
    from sparse_block_attention_amd import pipeline, synth
    res = {}
    scratch = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    total = torch.zeros((), dtype=torch.int64, device="cuda")

    def evict():
        torch.sum(scratch.view(torch.int32), dim=0, out=total)

    for name in names:
        w = synth.WORKLOADS[name]
        L, A, l, p = w.local_len, w.anchor_len, w.pass_per_host, w.host
        Hq, Hkv, d, Hs = w.n_q_heads, w.n_kv_heads, w.head_dim, w.hidden
        g = Hq // Hkv
        print(f"# workload {name}", file=sys.stderr, flush=True)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(1000 + w.config_id)

        def rnd(*shape, sigma=0.5):
            return (torch.randn(shape, generator=gen, device="cuda") * sigma).to(torch.bfloat16)

        pr = B.Problem(Hq, Hkv, d, L, A, l, p, w.n_hosts, None)
        host = pipeline.HostTensors(rnd(L, Hq, d), rnd(L, Hkv, d), rnd(L, Hkv, d))
        ka, va = (rnd(A, Hkv, d), rnd(A, Hkv, d)) if A else (None, None)
        kcs = [rnd(l, Hkv, d) for _ in range(p)]
        vcs = [rnd(l, Hkv, d) for _ in range(p)]
        sc = {"w1": rnd(Hkv, Hs, (g + 2) * d, sigma=0.1),
              "b1": torch.randn((Hkv, Hs), generator=gen, device="cuda") * 0.1,
              "w2": torch.randn((Hkv, Hs), generator=gen, device="cuda") * 0.1,
              "b2": torch.randn((Hkv,), generator=gen, device="cuda") * 0.1}
        buf = pipeline.StepBuffers.allocate(pr)
        byt = stage_bytes(w)
        fns = {
            "a1_score": lambda: B.apb_score_kv(pr, sc, host.q, host.k, host.v, scores=buf.scores),
            "a2a3_topl_gather": lambda: B.apb_topk_gather(pr, buf.scores, host.k, host.v, idx=buf.idx,
                                                          k_comp=buf.k_comp, v_comp=buf.v_comp,
                                                          workspace=buf.topk_workspace),
        }
        if pr.pass_len:
            fns["a5_passing"] = lambda: B.apb_build_passing(pr, kcs, vcs, k_pass=buf.k_pass, v_pass=buf.v_pass)
        r = {"config": {"local_len": L, "anchor_len": A, "pass_len": pr.pass_len, "n_q_heads": Hq,
                        "n_kv_heads": Hkv, "head_dim": d, "scorer_hidden": Hs}}
        for st, fn in fns.items():
            med, mn = _stage_times(fn, reps, warm)
            cmed, _ = _stage_times(fn, reps, warm, evict=evict)
            r[st] = {"us_median": med * 1e3, "us_min": mn * 1e3, "cold_us_median": cmed * 1e3, "bytes": byt[st],
                     "frac_hbm_peak": byt[st] / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "cold_frac_hbm_peak": byt[st] / (cmed * 1e-3) / 1e9 / PEAK_HBM_GBS}
        for tag, key in (("warm", "us_median"), ("cold", "cold_us_median")):
            t = r["a1_score"][key] + r["a2a3_topl_gather"][key]
            b = byt["a1_score"] + byt["a2a3_topl_gather"]
            r[tag + "_a1_a3"] = {"us_median": t, "frac_hbm_peak": b / (t * 1e-6) / 1e9 / PEAK_HBM_GBS}
        attn = lambda: B.apb_block_attention(pr, host.q, ka, va, buf.k_pass, buf.v_pass, host.k, host.v,
                                             out=buf.out, lse=buf.lse)
        if pr.pass_len:
            B.apb_build_passing(pr, kcs, vcs, k_pass=buf.k_pass, v_pass=buf.v_pass)
        n_att = 3 if L > 65536 else reps
        for _ in range(2):
            attn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_att)]
        for a, b in ev:
            a.record()
            attn()
            b.record()
        torch.cuda.synchronize()
        r["attention"] = _attention_stats([a.elapsed_time(b) for a, b in ev], attention_flops(w))
        t_step = (r["a1_score"]["us_median"] + r["a2a3_topl_gather"]["us_median"]
                  + (r["a5_passing"]["us_median"] if pr.pass_len else 0.0)) * 1e-3 + r["attention"]["ms"]
        r["prefill_tokens_per_s_serial_steps"] = L / (t_step * 1e-3)
        res[name] = r
        del host, ka, va, kcs, vcs, sc, buf
        torch.cuda.empty_cache()
    del scratch
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true",
                    help="run the host's compression on the same stream as its attention "
                         "instead of a second stream")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the split-phase and baseline-mode attention timings")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before warm-up, run one plain device-to-device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: it measures one host's block, and the exchange between "
              f"hosts is not part of this library (--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_block_attention_amd import binding as B
    from sparse_block_attention_amd import pipeline, synth
    from sparse_block_attention_amd.tensors import to_device_bf16, to_device_f32

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()
    w = synth.WORKLOADS[args.workload]
    pr = B.Problem(w.n_q_heads, w.n_kv_heads, w.head_dim, w.local_len, w.anchor_len,
                   w.pass_per_host, w.host, w.n_hosts, None)
    print(f"# generating {w.name} inputs", file=sys.stderr, flush=True)
    wts = synth.scorer_weights(w)
    sc = {"w1": to_device_bf16(wts["w1"]), "b1": to_device_f32(wts["b1"]),
          "w2": to_device_f32(wts["w2"]), "b2": to_device_f32(wts["b2"])}
    ka_np, va_np = synth.anchor_kv(w)
    ka = to_device_bf16(ka_np) if w.anchor_len else None
    va = to_device_bf16(va_np) if w.anchor_len else None
    kcs, vcs = [], []
    prior_kv = []
    host_np = None
    for j in range(w.host + 1):
        q, k, v = synth.host_block(w, j)
        ht = pipeline.HostTensors(to_device_bf16(q), to_device_bf16(k), to_device_bf16(v))
        if j < w.host:
            pj = B.Problem(w.n_q_heads, w.n_kv_heads, w.head_dim, w.local_len, w.anchor_len,
                           w.pass_per_host, j, w.n_hosts, None)
            _, _, kc, vc = pipeline.compress(pj, sc, ht)
            kcs.append(kc)
            vcs.append(vc)
            if not args.no_extras:
                prior_kv.append((ht.k, ht.v))
            del ht
        else:
            host = ht
            host_np = (q, k, v)
    torch.cuda.synchronize()
    buf = pipeline.StepBuffers.allocate(pr)
    stream = torch.cuda.current_stream()
    # The host's own compression is independent of its attention: a second stream
    # (default priority) lets the two overlap.
    side = None if args.serial else torch.cuda.Stream()
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print("# warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        pipeline.host_step(pr, sc, host, ka, va, kcs, vcs, buf, stream=stream, side_stream=side)
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    print("# timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        pipeline.host_step(pr, sc, host, ka, va, kcs, vcs, buf, stream=stream, attn_events=ev[i],
                           side_stream=side)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    attn_times = [a.elapsed_time(b) for a, b in ev]
    attn_ms = float(np.mean(attn_times))
    flops = attention_flops(w)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    traffic = measured_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": w.local_len / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {DESCRIPTIONS[w.name]}", "local_len": w.local_len,
                   "anchor_len": w.anchor_len, "pass_len": w.pass_len, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "scorer_hidden": w.hidden,
                   "host_index": w.host, "n_hosts": w.n_hosts},
        "attention": _attention_stats(attn_times, flops),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic},
    }
    if not args.no_extras:
        print("# each step alone, warm and cold", file=sys.stderr, flush=True)
        result["stages"] = stages(B, w, pr, sc, host, ka, va, kcs, vcs, buf)
        result["sclk_mhz_after"] = sclk_mhz()
    if not args.no_extras and prior_kv:
        print("# split-phase attention, steps either side, baseline modes", file=sys.stderr, flush=True)
        result["split_phase"] = split_phase(B, pr, host, ka, va, buf.k_pass, buf.v_pass, attn_ms)
        # The steps either side run before the baseline modes, whose 25 ms attention
        # launches would otherwise leave them on a GPU clocked down by the heat.
        result["layer_sides"] = layer_sides(B, w, host, ka, va)
        result["modes"] = baseline_modes(B, w, host, prior_kv, attn_ms)
    del buf, host, kcs, vcs, prior_kv
    if not args.no_extras:
        import torch as _t
        _t.cuda.empty_cache()
        others = [n for n in ("tiny", "qwen14b", "yi34b", "llama1m") if n != w.name]
        result["workloads"] = other_workloads(B, others)
        result["scorer_weight_bytes"] = scorer_weight_bytes(w)
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle on a bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, host_np, wts, (ka_np, va_np))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
