"""Thin Python binding of libdash (ctypes).  Argument marshalling only: every step of the
attention path runs in the library's HIP kernels.  PyTorch supplies device memory and the
current stream.

The keyword interface mirrors the one described for the authors' package (aiexpert.news
article, paragraph on the Triton release): queries, keys, values, a per-head
classification vector `head_cls`, `chunk_size`, `estimate_diagonal`, `enable_gqa`, and an
optional `active_blocks` mask.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdash.so")

DASH_OK = 0
ERRORS = {
    -1: "DASH_ERR_INVALID_ARG", -2: "DASH_ERR_SHAPE", -3: "DASH_ERR_DTYPE",
    -4: "DASH_ERR_UNSUPPORTED", -5: "DASH_ERR_WORKSPACE", -6: "DASH_ERR_HIP",
}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}

EXPORTS = [
    "dash_abi_version", "dash_last_error",
    "dash_prefill_workspace_size", "dash_prefill", "dash_prefill_stage",
    "dash_decode_workspace_size", "dash_decode", "dash_decode_diag", "dash_decode_noalloc",
    "dash_append_chunk", "dash_decode_paged", "dash_decode_paged_diag", "dash_append_chunk_paged",
    "dash_dense_causal_workspace_size", "dash_dense_causal",
    "dash_prefill_train", "dash_prefill_backward_workspace_size", "dash_prefill_backward",
]


class DashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class DashParams(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("gamma", ctypes.c_float), ("sm_scale", ctypes.c_float),
        ("enable_gqa", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("estimate_diagonal", ctypes.c_int32), ("sigma", ctypes.c_float),
        ("topk", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdash.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libdash.so not found at {path}; build it with "
                           "`python -m long_context_sparse_stage0_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(DashParams)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.dash_abi_version.restype = ctypes.c_int
    lib.dash_last_error.restype = ctypes.c_char_p
    for name in ("dash_prefill_workspace_size", "dash_decode_workspace_size",
                 "dash_dense_causal_workspace_size", "dash_prefill_backward_workspace_size"):
        f = getattr(lib, name)
        f.argtypes = [P, ctypes.POINTER(sz)]
        f.restype = ctypes.c_int
    lib.dash_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_prefill.restype = ctypes.c_int
    lib.dash_prefill_stage.argtypes = [P, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_prefill_stage.restype = ctypes.c_int
    lib.dash_decode.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_decode.restype = ctypes.c_int
    lib.dash_decode_diag.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_decode_diag.restype = ctypes.c_int
    lib.dash_decode_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dash_decode_noalloc.restype = ctypes.c_int
    lib.dash_append_chunk.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.dash_append_chunk.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.dash_decode_paged.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_decode_paged_diag.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_decode_paged_diag.restype = ctypes.c_int
    lib.dash_decode_paged.restype = ctypes.c_int
    lib.dash_append_chunk_paged.argtypes = [P, vp, i32, vp, vp, vp, vp, vp, vp]
    lib.dash_append_chunk_paged.restype = ctypes.c_int
    lib.dash_dense_causal.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_dense_causal.restype = ctypes.c_int
    lib.dash_prefill_train.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dash_prefill_train.restype = ctypes.c_int
    lib.dash_prefill_backward.argtypes = [P] + [vp] * 11 + [vp, sz, vp]
    lib.dash_prefill_backward.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != DASH_OK:
        raise DashError(rc, load().dash_last_error().decode())


def make_params(B, Hq, Hkv, T, D, *, chunk_size=64, alpha=1.5, gamma=1.0, sm_scale=None,
                enable_gqa=False, dtype=torch.bfloat16, estimate_diagonal=False,
                sigma=1.0, topk=0) -> DashParams:
    return DashParams(B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, chunk_size=chunk_size, alpha=alpha,
                      gamma=gamma, sm_scale=0.0 if sm_scale is None else sm_scale,
                      enable_gqa=int(bool(enable_gqa)), dtype=DTYPES.get(dtype, 99),
                      estimate_diagonal=int(bool(estimate_diagonal)), sigma=sigma, topk=topk)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(kind: str, params: DashParams) -> int:
    n = ctypes.c_size_t(0)
    f = {"prefill": load().dash_prefill_workspace_size,
         "decode": load().dash_decode_workspace_size,
         "dense": load().dash_dense_causal_workspace_size,
         "backward": load().dash_prefill_backward_workspace_size}[kind]
    _check(f(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def prefill(q, k, v, head_cls, *, chunk_size=64, alpha=1.5, gamma=1.0, sm_scale=None,
            sigma=1.0, topk=0, enable_gqa=False, estimate_diagonal=False,
            return_active_blocks=False,
            return_block_weights=False, return_summaries=False, out=None, workspace=None,
            stream=None):
    """Causal prefill.  q [B,Hq,T,D]; k, v [B,Hkv,T,D]; head_cls [Hkv,D].
    Returns out, followed by the requested extras in the order
    (active_blocks [B,Hkv,T,W] int64 bit-words, block_weights [B,Hkv,T,nc] fp32,
     summaries [B,Hkv,nc,D] fp32)."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    p = make_params(B, Hq, Hkv, T, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype,
                    estimate_diagonal=estimate_diagonal, sigma=sigma, topk=topk)
    nc = -(-T // 64)
    W = -(-nc // 64)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    ab = torch.empty((B, Hkv, T, W), dtype=torch.int64, device=dev) if return_active_blocks else None
    bw = torch.empty((B, Hkv, T, nc), dtype=torch.float32, device=dev) if return_block_weights else None
    sm = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device=dev) if return_summaries else None
    if workspace is None:
        workspace = alloc_workspace(workspace_size("prefill", p), dev)
    _check(load().dash_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(head_cls),
                               _ptr(out), _ptr(ab), _ptr(bw), _ptr(sm), _ptr(workspace),
                               workspace.numel(), _stream(stream)))
    extras = [x for x in (ab, bw, sm) if x is not None]
    return (out, *extras) if extras else out


def prefill_train(q, k, v, head_cls, *, chunk_size=64, alpha=1.5, gamma=1.0, sm_scale=None,
                  sigma=1.0, enable_gqa=False, out=None, lse=None, workspace=None, stream=None):
    """Causal prefill that also returns lse [B,Hq,T] fp32, the per-row log-sum-exp that
    `prefill_backward` needs.  Returns (out, lse)."""
    B, Hq, T, D = q.shape
    p = make_params(B, Hq, k.shape[1], T, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype, sigma=sigma)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size("prefill", p), q.device)
    _check(load().dash_prefill_train(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(head_cls),
                                     _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                     _stream(stream)))
    return out, lse


def prefill_backward(q, k, v, head_cls, out, dout, lse, *, chunk_size=64, alpha=1.5,
                     gamma=1.0, sm_scale=None, sigma=1.0, enable_gqa=False, workspace=None,
                     stream=None):
    """Gradients of L with dL/dout = dout through the whole prefill (the same parameters as
    the forward).  Returns (dq, dk, dv, dhead_cls); dhead_cls is fp32."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    p = make_params(B, Hq, Hkv, T, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype, sigma=sigma)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dhc = torch.empty((Hkv, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size("backward", p), q.device)
    _check(load().dash_prefill_backward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(head_cls), _ptr(out), _ptr(dout), _ptr(lse),
                                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dhc),
                                        _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv, dhc


def prefill_stage(stage, q, k, v, head_cls, out, workspace, *, alpha=1.5, gamma=1.0,
                  sm_scale=None, sigma=1.0, topk=0, enable_gqa=False, active_blocks=None,
                  block_weights=None, estimate_diagonal=False,
                  summaries=None, stream=None):
    """Run one prefill stage (0, 1 or 2) from the intermediates a full `prefill` call with
    the same tensors and workspace left behind (profiling aid)."""
    B, Hq, T, D = q.shape
    p = make_params(B, Hq, k.shape[1], T, D, alpha=alpha, gamma=gamma, sm_scale=sm_scale,
                    enable_gqa=enable_gqa, dtype=q.dtype, sigma=sigma, topk=topk,
                    estimate_diagonal=estimate_diagonal)
    _check(load().dash_prefill_stage(ctypes.byref(p), int(stage), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(head_cls), _ptr(out), _ptr(active_blocks),
                                     _ptr(block_weights), _ptr(summaries), _ptr(workspace),
                                     workspace.numel(), _stream(stream)))


def decode(q, k_cache, v_cache, seq_lens, summary_cache, *, chunk_size=64, alpha=1.5,
           gamma=1.0, sm_scale=None, sigma=1.0, topk=0, enable_gqa=False,
           estimate_diagonal=False, head_cls=None,
           return_active_blocks=False, out=None, workspace=None, stream=None):
    """One decode step.  q [B,Hq,D]; caches [B,Hkv,T_max,D]; seq_lens [B] int32 (device);
    summary_cache [B,Hkv,ceil(T_max/64),D] fp32.  estimate_diagonal needs head_cls [Hkv,D]
    (dash_decode_diag)."""
    B, Hq, D = q.shape
    Hkv, T_max = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, Hq, Hkv, T_max, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype, sigma=sigma,
                    topk=topk, estimate_diagonal=estimate_diagonal)
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    nc = -(-T_max // 64)
    W = -(-nc // 64)
    if out is None:
        out = torch.empty_like(q)
    ab = torch.empty((B, Hkv, W), dtype=torch.int64, device=q.device) if return_active_blocks else None
    if workspace is None:
        workspace = alloc_workspace(workspace_size("decode", p), q.device)
    if head_cls is not None:
        _check(load().dash_decode_diag(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(head_cls), _ptr(seq_lens), _ptr(summary_cache),
                                       _ptr(out), _ptr(ab), _ptr(workspace), workspace.numel(),
                                       _stream(stream)))
    else:
        _check(load().dash_decode(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(seq_lens), _ptr(summary_cache), _ptr(out), _ptr(ab),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out, ab) if return_active_blocks else out


def decode_noalloc(q, k_cache, v_cache, seq_lens, summary_cache, *, chunk_size=64, alpha=1.5,
                   gamma=1.0, sm_scale=None, sigma=1.0, topk=0, enable_gqa=False, out=None,
                   active_blocks=None, stream=None):
    """`decode` through dash_decode_noalloc: the library's fixed device scratch instead of a
    workspace, so the call allocates nothing itself (pass `out`, and `active_blocks` if
    wanted, preallocated).  Calls overlapping on one GPU race on that scratch."""
    B, Hq, D = q.shape
    Hkv, T_max = k_cache.shape[1], k_cache.shape[2]
    p = make_params(B, Hq, Hkv, T_max, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype, sigma=sigma,
                    topk=topk)
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    if out is None:
        out = torch.empty_like(q)
    _check(load().dash_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(seq_lens), _ptr(summary_cache), _ptr(out),
                                      _ptr(active_blocks), _stream(stream)))
    return out


def append_chunk(k_cache, head_cls, seq_lens, summary_cache, n_summarized, *, chunk_size=64,
                 sm_scale=None, enable_gqa=True, Hq=None, stream=None):
    """Summarise every newly completed chunk into summary_cache; advances n_summarized."""
    B, Hkv, T_max, D = k_cache.shape
    p = make_params(B, Hq if Hq is not None else Hkv, Hkv, T_max, D, chunk_size=chunk_size,
                    sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=k_cache.dtype)
    _check(load().dash_append_chunk(ctypes.byref(p), _ptr(k_cache), _ptr(head_cls),
                                    _ptr(seq_lens), _ptr(summary_cache), _ptr(n_summarized),
                                    _stream(stream)))


def _paged_params(q_or_none, k_pages, block_table, Hq, chunk_size, alpha, gamma, sm_scale,
                  sigma, enable_gqa, topk=0):
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise ValueError("block_table must be an int32 [B, ceil(T_max/64)] tensor")
    num_pages, Hkv, C, D = k_pages.shape
    if C != chunk_size:
        raise ValueError(f"pages must hold {chunk_size} tokens (got {C})")
    B = block_table.shape[0]
    T_max = block_table.shape[1] * chunk_size
    p = make_params(B, Hq, Hkv, T_max, D, chunk_size=chunk_size, alpha=alpha, gamma=gamma,
                    sm_scale=sm_scale, sigma=sigma, enable_gqa=enable_gqa, dtype=k_pages.dtype,
                    topk=topk)
    return p, num_pages


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, summary_cache, *, chunk_size=64,
                 alpha=1.5, gamma=1.0, sm_scale=None, sigma=1.0, topk=0, enable_gqa=False,
                 estimate_diagonal=False, head_cls=None,
                 return_active_blocks=False, out=None, workspace=None, stream=None):
    """One decode step over paged caches.  q [B,Hq,D]; k_pages, v_pages [num_pages,Hkv,64,D];
    block_table [B, ceil(T_max/64)] int32 (device); the rest as for `decode`."""
    B, Hq, D = q.shape
    p, num_pages = _paged_params(q, k_pages, block_table, Hq, chunk_size, alpha, gamma, sm_scale,
                                 sigma, enable_gqa, topk)
    p.estimate_diagonal = int(bool(estimate_diagonal))
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    W = -(-block_table.shape[1] // 64)
    if out is None:
        out = torch.empty_like(q)
    ab = torch.empty((B, k_pages.shape[1], W), dtype=torch.int64, device=q.device) \
        if return_active_blocks else None
    if workspace is None:
        workspace = alloc_workspace(workspace_size("decode", p), q.device)
    if head_cls is not None:
        _check(load().dash_decode_paged_diag(ctypes.byref(p), _ptr(q), _ptr(k_pages),
                                             _ptr(v_pages), num_pages, _ptr(block_table),
                                             _ptr(head_cls), _ptr(seq_lens), _ptr(summary_cache),
                                             _ptr(out), _ptr(ab), _ptr(workspace),
                                             workspace.numel(), _stream(stream)))
    else:
        _check(load().dash_decode_paged(ctypes.byref(p), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                        num_pages, _ptr(block_table), _ptr(seq_lens),
                                        _ptr(summary_cache), _ptr(out), _ptr(ab), _ptr(workspace),
                                        workspace.numel(), _stream(stream)))
    return (out, ab) if return_active_blocks else out


def append_chunk_paged(k_pages, block_table, head_cls, seq_lens, summary_cache, n_summarized, *,
                       chunk_size=64, sm_scale=None, enable_gqa=True, Hq=None, stream=None):
    """`append_chunk` over a paged K pool [num_pages, Hkv, 64, D] and its block table."""
    p, num_pages = _paged_params(None, k_pages, block_table,
                                 Hq if Hq is not None else k_pages.shape[1], chunk_size, 1.5,
                                 1.0, sm_scale, 1.0, enable_gqa)
    _check(load().dash_append_chunk_paged(ctypes.byref(p), _ptr(k_pages), num_pages,
                                          _ptr(block_table), _ptr(head_cls), _ptr(seq_lens),
                                          _ptr(summary_cache), _ptr(n_summarized),
                                          _stream(stream)))


def dense_causal(q, k, v, *, sm_scale=None, enable_gqa=False, out=None, workspace=None,
                 stream=None):
    """Dense causal softmax attention (the comparator), same layouts, bf16."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    p = make_params(B, Hq, Hkv, T, D, sm_scale=sm_scale, enable_gqa=enable_gqa, dtype=q.dtype)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(workspace_size("dense", p), q.device)
    _check(load().dash_dense_causal(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                    _ptr(workspace), workspace.numel(), _stream(stream)))
    return out
