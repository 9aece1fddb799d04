"""DashAttention backward pass -- plain float64 CPU oracle.

TEST INFRASTRUCTURE ONLY, like dash_oracle.py: only the tests, the smoke check and the
benchmark's CPU baseline may import or run it; the product never calls it.

The pages' central claim is that the whole hierarchy is differentiable end to end: the
routing distribution is alpha-entmax, whose Jacobian exists almost everywhere, so the
gradient of the loss reaches the query-summary scores and, through them, Stage 0's
classifier query and keys (gist.science summary of arXiv 2605.18753, "Stufe 1:
Entmax-Chunk-Routing", remark on differentiability, and "Hauptbeiträge"; aixai.ru blog,
the section on why top-k routing breaks gradients).  This file takes the forward of
dash_oracle.prefill backwards, step by step in reverse page order, for a loss L whose
gradient with respect to the output is `dout`:

  Stage 2 (per head and row; softmax(z + sigma log g) attention):
      P = softmax(l),  l_j = s <q, k_j> + beta_j,  o = sum_j P_j v_j
      dv_j += P_j dO;  dP_j = <dO, v_j>;  dl_j = P_j (dP_j - <dO, o>)
      dq += s sum_j dl_j k_j;  dk_j += s dl_j q;  dbeta_j = dl_j
      a routed chunk's bias is sigma log w_bar_c, so  dw_bar_c += sigma / w_bar_c *
      sum over the chunk's keys (and over the G heads sharing w_bar) of dl_j.
  GQA mean: w_bar = (1/G) sum_h p_h  ->  dp_h = dw_bar / G.
  alpha-entmax (Peters, Niculae and Martins 2019, the Jacobian of their Proposition on
      the entmax gradient): with s_i = p_i^(2 - alpha) on the support and 0 off it,
      dx = s * dp - s (s . dp) / (sum s).
  Stage 1 scores x_{h,c} = gamma s <q_h, k_bar_c>:
      dq_h += gamma s sum_c dx_{h,c} k_bar_c;  dk_bar_c += gamma s sum dx_{h,c} q_h.
  Stage 0 (k_bar = sum_j pi_j k_j, pi = softmax(a), a_j = s <hc, k_j>):
      dk_j += pi_j dk_bar;  da_j = pi_j (<dk_bar, k_j> - <dk_bar, k_bar>);
      dk_j += s da_j hc;  dhc += s sum_j da_j k_j.

Scope: the method's routing (alpha-entmax, estimate_diagonal off).  The diagonal chunk's
keys carry no bias, so no gradient reaches routing through them.  At a chunk whose entmax
argument sits exactly on the threshold the gradient is one-sided; every pin below keeps
such points out.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import dash_oracle as F

CHUNK = F.CHUNK


def entmax_backward(p: np.ndarray, dp: np.ndarray, alpha: float) -> np.ndarray:
    """Gradient with respect to x of alpha-entmax(x), given p = entmax(x) and dL/dp,
    along the last axis: s = p^(2 - alpha) on the support, dx = s dp - s (s.dp)/sum s."""
    p = np.asarray(p, np.float64)
    dp = np.asarray(dp, np.float64)
    s = np.where(p > 0.0, np.power(np.where(p > 0.0, p, 1.0), 2.0 - alpha), 0.0)
    ss = s.sum(axis=-1, keepdims=True)
    return s * dp - s * (s * dp).sum(axis=-1, keepdims=True) / ss


def chunk_summaries_backward(k: np.ndarray, head_cls: np.ndarray, scale: float,
                             dsumm: np.ndarray, chunk: int = CHUNK):
    """Stage 0 backwards.  k [B, Hkv, T, D], head_cls [Hkv, D], dsumm [B, Hkv, nf, D]
    (gradient for the summaries of the nf complete chunks).  Returns (dk, dhead_cls)."""
    k = np.asarray(k, np.float64)
    hc = np.asarray(head_cls, np.float64)
    B, H, T, D = k.shape
    nf = T // chunk
    dk = np.zeros_like(k)
    dhc = np.zeros_like(hc)
    for b in range(B):
        for h in range(H):
            for c in range(nf):
                kc = k[b, h, c * chunk:(c + 1) * chunk]
                a = scale * (kc @ hc[h])
                pi = F.softmax(a)
                kbar = pi @ kc
                g = np.asarray(dsumm[b, h, c], np.float64)
                dk[b, h, c * chunk:(c + 1) * chunk] += np.outer(pi, g)
                da = pi * (kc @ g - kbar @ g)
                dk[b, h, c * chunk:(c + 1) * chunk] += scale * np.outer(da, hc[h])
                dhc[h] += scale * (da @ kc)
    return dk, dhc


def attend_row_backward(q, k, v, t, w_bar, dout, *, scale, sigma=1.0, chunk=CHUNK):
    """Stage 2 backwards for one head at row t (the keys and biases of
    dash_oracle.attend_row).  Returns (dq [D], dk [t+1, D], dv [t+1, D], dwb [t // C]):
    dwb_c is the gradient with respect to w_bar_c through this head's biases."""
    it = t // chunk
    idx, bias, chunk_of = [], [], []
    for c in range(it):
        if w_bar[c] > 0.0:
            idx.extend(range(c * chunk, (c + 1) * chunk))
            bias.extend([sigma * math.log(w_bar[c])] * chunk)
            chunk_of.extend([c] * chunk)
    idx.extend(range(it * chunk, t + 1))
    bias.extend([0.0] * (t + 1 - it * chunk))
    chunk_of.extend([-1] * (t + 1 - it * chunk))
    idx = np.asarray(idx)
    chunk_of = np.asarray(chunk_of)
    qq = np.asarray(q, np.float64)
    kk = np.asarray(k[idx], np.float64)
    vv = np.asarray(v[idx], np.float64)
    do = np.asarray(dout, np.float64)
    logits = scale * (kk @ qq) + np.asarray(bias)
    P = F.softmax(logits)
    o = P @ vv
    dP = vv @ do
    dl = P * (dP - do @ o)
    dq = scale * (dl @ kk)
    dk = np.zeros((t + 1, qq.size))
    dv = np.zeros((t + 1, qq.size))
    dk[idx] += scale * np.outer(dl, qq)
    dv[idx] += np.outer(P, do)
    dwb = np.zeros(it)
    routed = chunk_of >= 0
    if it > 0 and routed.any():
        per_chunk = np.bincount(chunk_of[routed], weights=dl[routed], minlength=it)
        on = w_bar > 0.0
        dwb[on] = sigma * per_chunk[on] / w_bar[on]
    return dq, dk, dv, dwb


def prefill_backward(q, k, v, head_cls, dout, *, alpha: float = 1.5, gamma: float = 1.0,
                     scale: Optional[float] = None, sigma: float = 1.0,
                     chunk: int = CHUNK) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(dout * prefill(q, k, v, head_cls)["out"]) with respect to q
    [B, Hq, T, D], k, v [B, Hkv, T, D] and head_cls [Hkv, D], in float64.  Also returns
    the gradient of the summaries ("dsumm") and of the head-averaged block weights
    ("dw_bar" [B, Hkv, T, n_c], zero where the block is inactive)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hc = np.asarray(head_cls, np.float64)
    dout = np.asarray(dout, np.float64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nc = -(-T // chunk)
    summ = F.chunk_summaries(k, hc, scale, chunk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsumm = np.zeros_like(summ)
    dwbar_all = np.zeros((B, Hkv, T, nc))
    for b in range(B):
        for kvh in range(Hkv):
            kk, vv = k[b, kvh], v[b, kvh]
            for t in range(T):
                qg = q[b, kvh * G:(kvh + 1) * G, t]
                wb, _, p = F.route_row(qg, summ[b, kvh], t, alpha=alpha, gamma=gamma,
                                       scale=scale, chunk=chunk)
                it = t // chunk
                dwb = np.zeros(it)
                for g in range(G):
                    h = kvh * G + g
                    dq_h, dk_h, dv_h, dwb_h = attend_row_backward(
                        qg[g], kk, vv, t, wb, dout[b, h, t], scale=scale, sigma=sigma,
                        chunk=chunk)
                    dq[b, h, t] += dq_h
                    dk[b, kvh, :t + 1] += dk_h
                    dv[b, kvh, :t + 1] += dv_h
                    dwb += dwb_h
                if it == 0:
                    continue
                dwbar_all[b, kvh, t, :it] = dwb
                # GQA mean, then each head's entmax, then its scores
                dp = np.broadcast_to(dwb / G, (G, it))
                dx = entmax_backward(p, dp, alpha)          # [G, it]
                dq[b, kvh * G:(kvh + 1) * G, t] += gamma * scale * (dx @ summ[b, kvh, :it])
                dsumm[b, kvh, :it] += gamma * scale * (dx.T @ qg)
    dk0, dhc = chunk_summaries_backward(k, hc, scale, dsumm, chunk)
    dk += dk0
    return {"dq": dq, "dk": dk, "dv": dv, "dhead_cls": dhc, "dsumm": dsumm,
            "dw_bar": dwbar_all}


def loss(q, k, v, head_cls, dout, **kw) -> float:
    """L = sum(dout * out): the scalar whose gradients prefill_backward returns."""
    out = F.prefill(q, k, v, head_cls, **kw)["out"]
    return float((np.asarray(dout, np.float64) * out).sum())
