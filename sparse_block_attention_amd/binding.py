"""ctypes binding of libapb.so: the C-ABI entry points under the same names.

Argument marshalling only: shapes, dtypes, devices and contiguity are checked,
outputs are allocated with torch when the caller passes none, and raw device
pointers plus the current HIP stream go to the library.  Every step of the
path runs in the library's HIP kernels; there is no fallback.  If libapb.so
is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_void_p
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libapb.so")

APB_OK = 0
APB_ERR_INVALID_ARGUMENT = 1
APB_ERR_UNSUPPORTED = 2
APB_ERR_WORKSPACE_TOO_SMALL = 3
APB_ERR_HIP = 4
APB_ERR_INTERNAL = 5

NOALLOC_TOPK_WORKSPACE_BYTES = 4 << 20   # APB_NOALLOC_TOPK_WORKSPACE_BYTES

APB_SEG_ANCHOR = 1
APB_SEG_PASSING = 2
APB_SEG_LOCAL = 4
APB_SEG_ALL = 7


class ApbError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {apb_status_string(status)}: {detail}")


class _Problem(ctypes.Structure):
    _fields_ = [("n_q_heads", c_int32), ("n_kv_heads", c_int32), ("head_dim", c_int32),
                ("local_len", c_int32), ("anchor_len", c_int32), ("pass_per_host", c_int32),
                ("host_index", c_int32), ("n_hosts", c_int32), ("kv_head_of_q", POINTER(c_int32))]


class _Scorer(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("w1", c_void_p), ("b1", c_void_p), ("w2", c_void_p),
                ("b2", c_void_p)]


@dataclass
class Problem:
    """One host's share of the evenly split sequence (fields of apb_problem)."""

    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    local_len: int
    anchor_len: int
    pass_per_host: int
    host_index: int
    n_hosts: int
    kv_head_of_q: Optional[Sequence[int]] = None

    @property
    def pass_len(self) -> int:
        return self.host_index * self.pass_per_host

    def to_c(self):
        """(ctypes struct, keep-alive array) for a call.  The library reads n_q_heads
        entries of the head map, so a map of any other length is refused here."""
        arr = None
        ptr = None
        if self.kv_head_of_q is not None:
            if len(self.kv_head_of_q) != self.n_q_heads:
                raise ValueError(f"kv_head_of_q has {len(self.kv_head_of_q)} entries, "
                                 f"need n_q_heads = {self.n_q_heads}")
            arr = (c_int32 * len(self.kv_head_of_q))(*[int(x) for x in self.kv_head_of_q])
            ptr = ctypes.cast(arr, POINTER(c_int32))
        s = _Problem(self.n_q_heads, self.n_kv_heads, self.head_dim, self.local_len,
                     self.anchor_len, self.pass_per_host, self.host_index, self.n_hosts, ptr)
        return s, arr


_lib = None


def lib() -> ctypes.CDLL:
    """Load libapb.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_block_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = POINTER(_Problem)
        L.apb_score_kv.argtypes = [P, POINTER(_Scorer), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.apb_topk_gather.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, ctypes.c_size_t, c_void_p]
        L.apb_topk_gather_noalloc.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p, c_void_p]
        L.apb_topk_workspace_size.argtypes = [P]
        L.apb_topk_workspace_size.restype = ctypes.c_size_t
        L.apb_build_passing.argtypes = [P, POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_void_p,
                                        c_void_p]
        L.apb_block_attention.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_float, c_void_p, c_void_p, c_void_p]
        L.apb_block_attention_segments.argtypes = [P, ctypes.c_uint32, c_void_p, c_void_p, c_void_p,
                                                   c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                                   c_void_p, c_void_p, c_void_p]
        L.apb_merge_attention.argtypes = [P, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p]
        L.apb_anchor_attention.argtypes = [P, c_void_p, c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                           c_void_p]
        L.apb_rope.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int32, ctypes.c_int64, c_float,
                               c_void_p]
        L.apb_qkv_projection.argtypes = [P, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p]
        L.apb_validate_problem.argtypes = [P]
        L.apb_status_string.argtypes = [c_int]
        L.apb_status_string.restype = c_char_p
        L.apb_last_error.argtypes = []
        L.apb_last_error.restype = c_char_p
        L.apb_abi_version.argtypes = []
        for name in ("apb_score_kv", "apb_topk_gather", "apb_topk_gather_noalloc", "apb_build_passing",
                     "apb_block_attention", "apb_block_attention_segments", "apb_merge_attention", "apb_anchor_attention",
                     "apb_rope", "apb_qkv_projection", "apb_validate_problem", "apb_abi_version"):
            getattr(L, name).restype = c_int
        _lib = L
    return _lib


def _check(status: int, func: str):
    if status != APB_OK:
        raise ApbError(status, func, lib().apb_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype, shape) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def apb_score_kv(problem: Problem, scorer: dict, q_local, k_local, v_local, scores=None, stream=None):
    """Scores fp32 [Hkv, L] (see apb_score_kv in include/apb.h)."""
    pr = problem
    L, Hq, Hkv, d = pr.local_len, pr.n_q_heads, pr.n_kv_heads, pr.head_dim
    g = Hq // Hkv
    w1 = scorer["w1"]
    Hs = int(w1.shape[1])
    if scores is None:
        scores = torch.empty((Hkv, L), dtype=torch.float32, device=q_local.device)
    sc = _Scorer(Hs, _ptr(w1, "w1", torch.bfloat16, (Hkv, Hs, (g + 2) * d)),
                 _ptr(scorer["b1"], "b1", torch.float32, (Hkv, Hs)),
                 _ptr(scorer["w2"], "w2", torch.float32, (Hkv, Hs)),
                 _ptr(scorer["b2"], "b2", torch.float32, (Hkv,)))
    cp, keep = pr.to_c()
    st = lib().apb_score_kv(ctypes.byref(cp), ctypes.byref(sc),
                            _ptr(q_local, "q_local", torch.bfloat16, (L, Hq, d)),
                            _ptr(k_local, "k_local", torch.bfloat16, (L, Hkv, d)),
                            _ptr(v_local, "v_local", torch.bfloat16, (L, Hkv, d)),
                            _ptr(scores, "scores", torch.float32, (Hkv, L)), _stream(stream))
    del keep
    _check(st, "apb_score_kv")
    return scores


def apb_topk_workspace_size(problem: Problem) -> int:
    """Bytes of workspace apb_topk_gather needs (0 for l == 0 or an invalid problem)."""
    cp, keep = problem.to_c()
    n = lib().apb_topk_workspace_size(ctypes.byref(cp))
    del keep
    return int(n)


def topk_workspace(problem: Problem, device="cuda") -> torch.Tensor:
    """A uint8 device tensor of apb_topk_workspace_size(problem) bytes (at least 1)."""
    return torch.empty(max(apb_topk_workspace_size(problem), 1), dtype=torch.uint8, device=device)


def apb_topk_gather(problem: Problem, scores, k_local, v_local, idx=None, k_comp=None, v_comp=None,
                    workspace=None, stream=None):
    """(idx int32 [Hkv, l], k_comp, v_comp bf16 [l, Hkv, d]) (see include/apb.h).

    `workspace` is a uint8 device tensor of at least apb_topk_workspace_size(problem)
    bytes; None allocates one for this call."""
    pr = problem
    L, Hkv, d, l = pr.local_len, pr.n_kv_heads, pr.head_dim, pr.pass_per_host
    dev = scores.device
    if idx is None:
        idx = torch.empty((Hkv, l), dtype=torch.int32, device=dev)
    if k_comp is None:
        k_comp = torch.empty((l, Hkv, d), dtype=torch.bfloat16, device=dev)
    if v_comp is None:
        v_comp = torch.empty((l, Hkv, d), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = topk_workspace(pr, dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" \
            or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the GPU")
    cp, keep = pr.to_c()
    st = lib().apb_topk_gather(ctypes.byref(cp), _ptr(scores, "scores", torch.float32, (Hkv, L)),
                               _ptr(k_local, "k_local", torch.bfloat16, (L, Hkv, d)),
                               _ptr(v_local, "v_local", torch.bfloat16, (L, Hkv, d)),
                               _ptr(idx, "idx", torch.int32, (Hkv, l)),
                               _ptr(k_comp, "k_comp", torch.bfloat16, (l, Hkv, d)),
                               _ptr(v_comp, "v_comp", torch.bfloat16, (l, Hkv, d)),
                               workspace.data_ptr(), workspace.numel(), _stream(stream))
    del keep
    _check(st, "apb_topk_gather")
    return idx, k_comp, v_comp


def apb_topk_gather_noalloc(problem: Problem, scores, k_local, v_local, idx, k_comp, v_comp, stream=None):
    """apb_topk_gather with the library's static per-GPU workspace (see include/apb.h).
    The caller passes every output; nothing is allocated here or in the library."""
    pr = problem
    L, Hkv, d, l = pr.local_len, pr.n_kv_heads, pr.head_dim, pr.pass_per_host
    cp, keep = pr.to_c()
    st = lib().apb_topk_gather_noalloc(ctypes.byref(cp), _ptr(scores, "scores", torch.float32, (Hkv, L)),
                                       _ptr(k_local, "k_local", torch.bfloat16, (L, Hkv, d)),
                                       _ptr(v_local, "v_local", torch.bfloat16, (L, Hkv, d)),
                                       _ptr(idx, "idx", torch.int32, (Hkv, l)),
                                       _ptr(k_comp, "k_comp", torch.bfloat16, (l, Hkv, d)),
                                       _ptr(v_comp, "v_comp", torch.bfloat16, (l, Hkv, d)), _stream(stream))
    del keep
    _check(st, "apb_topk_gather_noalloc")
    return idx, k_comp, v_comp


def apb_build_passing(problem: Problem, k_comps, v_comps, k_pass=None, v_pass=None, stream=None):
    """(k_pass, v_pass) bf16 [p*l, Hkv, d] from p compressed blocks (see include/apb.h)."""
    pr = problem
    p, l, Hkv, d = pr.host_index, pr.pass_per_host, pr.n_kv_heads, pr.head_dim
    P = p * l
    if len(k_comps) != p or len(v_comps) != p:
        raise ValueError(f"need {p} compressed blocks for host {p}, got {len(k_comps)}/{len(v_comps)}")
    dev = k_comps[0].device if p else torch.device("cuda")
    if k_pass is None:
        k_pass = torch.empty((P, Hkv, d), dtype=torch.bfloat16, device=dev)
    if v_pass is None:
        v_pass = torch.empty((P, Hkv, d), dtype=torch.bfloat16, device=dev)
    kh = (c_void_p * max(p, 1))(*[_ptr(t, f"k_comps[{j}]", torch.bfloat16, (l, Hkv, d))
                                 for j, t in enumerate(k_comps)])
    vh = (c_void_p * max(p, 1))(*[_ptr(t, f"v_comps[{j}]", torch.bfloat16, (l, Hkv, d))
                                 for j, t in enumerate(v_comps)])
    cp, keep = pr.to_c()
    st = lib().apb_build_passing(ctypes.byref(cp), kh, vh,
                                 _ptr(k_pass, "k_pass", torch.bfloat16, (P, Hkv, d)),
                                 _ptr(v_pass, "v_pass", torch.bfloat16, (P, Hkv, d)), _stream(stream))
    del keep
    _check(st, "apb_build_passing")
    return k_pass, v_pass


def _attention_outputs(problem: Problem, dev, out, lse):
    L, Hq, d = problem.local_len, problem.n_q_heads, problem.head_dim
    if out is None:
        out = torch.empty((L, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is True:
        lse = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    elif lse is False:
        lse = None
    return out, lse


def apb_block_attention_segments(problem: Problem, segments: int, q_local, k_anchor, v_anchor,
                                 k_pass, v_pass, k_local, v_local,
                                 softmax_scale: Optional[float] = None, out=None, lse=True,
                                 stream=None):
    """Attention over the key segments in `segments` (OR of APB_SEG_*; see include/apb.h).

    Returns (out bf16 [L, Hq, d], lse fp32 [Hq, L] or None).  Tensors of segments
    left out are ignored and may be None.  lse=True allocates the log-sum-exp
    output, lse=None/False skips it, a tensor is used as is.
    """
    pr = problem
    L, Hq, Hkv, d = pr.local_len, pr.n_q_heads, pr.n_kv_heads, pr.head_dim
    use_a, use_p, use_l = (segments & APB_SEG_ANCHOR, segments & APB_SEG_PASSING,
                           segments & APB_SEG_LOCAL)
    A = pr.anchor_len if use_a else 0
    P = pr.pass_len if use_p else 0
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out, lse = _attention_outputs(pr, q_local.device, out, lse)

    def seg(t, name, rows, used):
        return _ptr(t, name, torch.bfloat16, (rows, Hkv, d)) if used else None

    cp, keep = pr.to_c()
    st = lib().apb_block_attention_segments(
        ctypes.byref(cp), int(segments), _ptr(q_local, "q_local", torch.bfloat16, (L, Hq, d)),
        seg(k_anchor, "k_anchor", A, A > 0), seg(v_anchor, "v_anchor", A, A > 0),
        seg(k_pass, "k_pass", P, P > 0), seg(v_pass, "v_pass", P, P > 0),
        seg(k_local, "k_local", L, use_l), seg(v_local, "v_local", L, use_l),
        float(softmax_scale), _ptr(out, "out", torch.bfloat16, (L, Hq, d)),
        _ptr(lse, "lse", torch.float32, (Hq, L)), _stream(stream))
    del keep
    _check(st, "apb_block_attention_segments")
    return out, lse


def apb_block_attention(problem: Problem, q_local, k_anchor, v_anchor, k_pass, v_pass, k_local,
                        v_local, softmax_scale: Optional[float] = None, out=None, lse=True,
                        stream=None):
    """(out bf16 [L, Hq, d], lse fp32 [Hq, L] or None) (see include/apb.h).

    lse=True allocates the log-sum-exp output, lse=None/False skips it, a tensor is used as is.
    """
    pr = problem
    L, A, P = pr.local_len, pr.anchor_len, pr.pass_len
    Hq, Hkv, d = pr.n_q_heads, pr.n_kv_heads, pr.head_dim
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    out, lse = _attention_outputs(pr, q_local.device, out, lse)
    cp, keep = pr.to_c()
    st = lib().apb_block_attention(
        ctypes.byref(cp), _ptr(q_local, "q_local", torch.bfloat16, (L, Hq, d)),
        _ptr(k_anchor, "k_anchor", torch.bfloat16, (A, Hkv, d)),
        _ptr(v_anchor, "v_anchor", torch.bfloat16, (A, Hkv, d)),
        _ptr(k_pass, "k_pass", torch.bfloat16, (P, Hkv, d)),
        _ptr(v_pass, "v_pass", torch.bfloat16, (P, Hkv, d)),
        _ptr(k_local, "k_local", torch.bfloat16, (L, Hkv, d)),
        _ptr(v_local, "v_local", torch.bfloat16, (L, Hkv, d)), float(softmax_scale),
        _ptr(out, "out", torch.bfloat16, (L, Hq, d)),
        _ptr(lse, "lse", torch.float32, (Hq, L)), _stream(stream))
    del keep
    _check(st, "apb_block_attention")
    return out, lse


def apb_merge_attention(problem: Problem, out_a, lse_a, out_b, lse_b, out=None, lse=True,
                        stream=None):
    """Merge two partial results over disjoint key sets (see include/apb.h).

    Returns (out bf16 [L, Hq, d], lse fp32 [Hq, L] or None).  `out` / `lse` may be
    out_a / lse_a (or the b side) to merge in place.
    """
    pr = problem
    L, Hq, d = pr.local_len, pr.n_q_heads, pr.head_dim
    out, lse = _attention_outputs(pr, out_a.device, out, lse)
    cp, keep = pr.to_c()
    st = lib().apb_merge_attention(
        ctypes.byref(cp), _ptr(out_a, "out_a", torch.bfloat16, (L, Hq, d)),
        _ptr(lse_a, "lse_a", torch.float32, (Hq, L)),
        _ptr(out_b, "out_b", torch.bfloat16, (L, Hq, d)),
        _ptr(lse_b, "lse_b", torch.float32, (Hq, L)),
        _ptr(out, "out", torch.bfloat16, (L, Hq, d)),
        _ptr(lse, "lse", torch.float32, (Hq, L)), _stream(stream))
    del keep
    _check(st, "apb_merge_attention")
    return out, lse


def apb_anchor_attention(problem: Problem, q_anchor, k_anchor, v_anchor,
                         softmax_scale: Optional[float] = None, out=None, lse=True, stream=None):
    """Causal attention of the anchor's queries over the anchor (see include/apb.h).

    Returns (out bf16 [A, Hq, d], lse fp32 [Hq, A] or None).
    """
    pr = problem
    A, Hq, Hkv, d = pr.anchor_len, pr.n_q_heads, pr.n_kv_heads, pr.head_dim
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    dev = q_anchor.device
    if out is None:
        out = torch.empty((A, Hq, d), dtype=torch.bfloat16, device=dev)
    if lse is True:
        lse = torch.empty((Hq, A), dtype=torch.float32, device=dev)
    elif lse is False:
        lse = None
    cp, keep = pr.to_c()
    st = lib().apb_anchor_attention(
        ctypes.byref(cp), _ptr(q_anchor, "q_anchor", torch.bfloat16, (A, Hq, d)),
        _ptr(k_anchor, "k_anchor", torch.bfloat16, (A, Hkv, d)),
        _ptr(v_anchor, "v_anchor", torch.bfloat16, (A, Hkv, d)), float(softmax_scale),
        _ptr(out, "out", torch.bfloat16, (A, Hq, d)), _ptr(lse, "lse", torch.float32, (Hq, A)),
        _stream(stream))
    del keep
    _check(st, "apb_anchor_attention")
    return out, lse


def apb_rope(x, pos0: int, theta_base: float, out=None, stream=None):
    """Rotary position embedding of bf16 x [rows, heads, d] (see include/apb.h); out may be x."""
    if x.dim() != 3:
        raise ValueError("x must be [rows, heads, head_dim]")
    rows, heads, d = (int(n) for n in x.shape)
    if out is None:
        out = torch.empty_like(x)
    st = lib().apb_rope(_ptr(x, "x", torch.bfloat16, (rows, heads, d)),
                        _ptr(out, "out", torch.bfloat16, (rows, heads, d)), rows, heads, d, int(pos0),
                        float(theta_base), _stream(stream))
    _check(st, "apb_rope")
    return out


def apb_qkv_projection(problem: Problem, x, wq, wk, wv, q=None, k=None, v=None, stream=None):
    """q, k, v of hidden states x [rows, hidden] (see include/apb.h): (q, k, v) bf16."""
    pr = problem
    Hq, Hkv, d = pr.n_q_heads, pr.n_kv_heads, pr.head_dim
    rows, hidden = (int(n) for n in x.shape)
    dev = x.device
    if q is None:
        q = torch.empty((rows, Hq, d), dtype=torch.bfloat16, device=dev)
    if k is None:
        k = torch.empty((rows, Hkv, d), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((rows, Hkv, d), dtype=torch.bfloat16, device=dev)
    cp, keep = pr.to_c()
    st = lib().apb_qkv_projection(
        ctypes.byref(cp), rows, hidden, _ptr(x, "x", torch.bfloat16, (rows, hidden)),
        _ptr(wq, "wq", torch.bfloat16, (Hq * d, hidden)), _ptr(wk, "wk", torch.bfloat16, (Hkv * d, hidden)),
        _ptr(wv, "wv", torch.bfloat16, (Hkv * d, hidden)), _ptr(q, "q", torch.bfloat16, (rows, Hq, d)),
        _ptr(k, "k", torch.bfloat16, (rows, Hkv, d)), _ptr(v, "v", torch.bfloat16, (rows, Hkv, d)),
        _stream(stream))
    del keep
    _check(st, "apb_qkv_projection")
    return q, k, v


def apb_validate_problem(problem: Problem) -> int:
    cp, keep = problem.to_c()
    st = lib().apb_validate_problem(ctypes.byref(cp))
    del keep
    return st


def apb_status_string(status: int) -> str:
    return lib().apb_status_string(int(status)).decode()


def apb_last_error() -> str:
    return lib().apb_last_error().decode()


def apb_abi_version() -> int:
    return lib().apb_abi_version()
