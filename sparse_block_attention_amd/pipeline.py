"""One host's share of one layer, run through the C-ABI entry points.

    score (apb_score_kv) -> top-l + gather (apb_topk_gather)
        -> passing block (apb_build_passing) -> attention (apb_block_attention)

The compressed blocks of the preceding hosts are passed in: on one GPU they
are produced by running the compression steps on those hosts' blocks into
device buffers, in place of the all-gather between hosts.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding as B


@dataclass
class HostTensors:
    """Device inputs of one host's block: q [L,Hq,d], k/v [L,Hkv,d] (bf16)."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor


def problem_for(n_q_heads, n_kv_heads, head_dim, local_len, anchor_len, pass_per_host, host_index,
                n_hosts, kv_head_of_q=None) -> B.Problem:
    return B.Problem(n_q_heads, n_kv_heads, head_dim, local_len, anchor_len, pass_per_host,
                     host_index, n_hosts, kv_head_of_q)


def compress(problem: B.Problem, scorer: dict, host: HostTensors, stream=None, workspace=None):
    """(scores, idx, k_comp, v_comp) of one host's block."""
    scores = B.apb_score_kv(problem, scorer, host.q, host.k, host.v, stream=stream)
    idx, kc, vc = B.apb_topk_gather(problem, scores, host.k, host.v, workspace=workspace, stream=stream)
    return scores, idx, kc, vc


@dataclass
class StepBuffers:
    """Preallocated outputs of one host step, reused across steps."""

    scores: torch.Tensor
    idx: torch.Tensor
    k_comp: torch.Tensor
    v_comp: torch.Tensor
    k_pass: Optional[torch.Tensor]
    v_pass: Optional[torch.Tensor]
    out: torch.Tensor
    lse: torch.Tensor
    topk_workspace: torch.Tensor

    @staticmethod
    def allocate(problem: B.Problem, device="cuda") -> "StepBuffers":
        L, Hq, Hkv, d = problem.local_len, problem.n_q_heads, problem.n_kv_heads, problem.head_dim
        l, P = problem.pass_per_host, problem.pass_len
        bf, f32 = torch.bfloat16, torch.float32
        return StepBuffers(
            scores=torch.empty((Hkv, L), dtype=f32, device=device),
            idx=torch.empty((Hkv, l), dtype=torch.int32, device=device),
            k_comp=torch.empty((l, Hkv, d), dtype=bf, device=device),
            v_comp=torch.empty((l, Hkv, d), dtype=bf, device=device),
            k_pass=torch.empty((P, Hkv, d), dtype=bf, device=device) if P else None,
            v_pass=torch.empty((P, Hkv, d), dtype=bf, device=device) if P else None,
            out=torch.empty((L, Hq, d), dtype=bf, device=device),
            lse=torch.empty((Hq, L), dtype=f32, device=device),
            topk_workspace=B.topk_workspace(problem, device))


def host_step(problem: B.Problem, scorer: dict, host: HostTensors, k_anchor, v_anchor,
              k_comps: List[torch.Tensor], v_comps: List[torch.Tensor], buf: StepBuffers,
              softmax_scale=None, stream=None, attn_events=None, side_stream=None) -> StepBuffers:
    """The whole per-host path into `buf`.  `attn_events` = (start, end) HIP events
    recorded around the attention launch on the same stream, or None.

    The host's own compression (score, top-l, gather) feeds the later hosts, not
    this host's attention, so with `side_stream` it runs there, concurrently with
    the passing build and the attention on `stream`; the call returns with
    `stream` made to wait for it, so the whole step is ordered before anything
    enqueued on `stream` afterwards.  Both streams keep the default priority.
    """
    main = stream if stream is not None else torch.cuda.current_stream()
    comp = side_stream if side_stream is not None else main
    if side_stream is not None:
        side_stream.wait_stream(main)          # inputs of this step are ready
    B.apb_score_kv(problem, scorer, host.q, host.k, host.v, scores=buf.scores, stream=comp)
    B.apb_topk_gather(problem, buf.scores, host.k, host.v, idx=buf.idx, k_comp=buf.k_comp,
                      v_comp=buf.v_comp, workspace=buf.topk_workspace, stream=comp)
    if problem.pass_len:
        B.apb_build_passing(problem, k_comps, v_comps, k_pass=buf.k_pass, v_pass=buf.v_pass,
                            stream=main)
    if attn_events is not None:
        attn_events[0].record(main)
    B.apb_block_attention(problem, host.q, k_anchor, v_anchor, buf.k_pass, buf.v_pass, host.k,
                          host.v, softmax_scale, out=buf.out, lse=buf.lse, stream=main)
    if attn_events is not None:
        attn_events[1].record(main)
    if side_stream is not None:
        main.wait_stream(side_stream)          # the step ends when both halves have
    return buf
