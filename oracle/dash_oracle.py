"""DashAttention forward pass -- plain float64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU
baseline may import or run anything in this directory.  It shares no code, constants or
helpers with the HIP library; the product never calls it.

What it computes, step by step, with the passage each step follows:

  Stage 0 (gist.science summary of arXiv 2605.18753, "Methodik", "Stufe 0: Lokale
  Chunk-Zusammenfassung"; liuzhao09 reading note, section 2): the keys are cut into
  contiguous chunks of C = 64; a learned per-head query q_bar attends, by scaled
  dot-product attention, over the keys of each chunk, and the attention-weighted key is
  the chunk summary.  With q_bar = 0 this is mean pooling.  Keys double as the values
  of this local attention (the pages say q_bar attends "over the keys").

  Stage 1 ("Stufe 1: Entmax-Chunk-Routing"): logits z_bar of each query against the
  chunk summaries; w_hat = alpha-entmax(gamma * z_bar).  In GQA the routing
  probabilities of the query heads that share a KV head are averaged into one shared
  sparse support.  alpha-entmax is the Tsallis-entropy transform of Peters, Niculae and
  Martins (2019, "Sparse Sequence-to-Sequence Models"):
      entmax_a(x) = argmax_{p in simplex} p.x + sum_j (p_j - p_j^a) / (a (a - 1)),
  whose solution is  p_j = [(a - 1) x_j - tau]_+ ^ (1 / (a - 1)),  tau fixed by sum p = 1.

  Stage 2 ("Stufe 2: Prior-induzierte spärliche Softmax"): softmax is the maximiser of
  z.p - KL(p || u); replacing the uniform u by a reference g derived from the routing
  weights, with g = 0 wherever w = 0, gives  p = g * exp(z) / sum(g * exp(z))
  = softmax(z + log g).  The query's own chunk, which has no summary yet, is a separate
  branch.  The pages name a prior-strength sigma without giving its form.

Readings taken where the pages are silent (each is one named argument or branch here):
  * summaries come only from complete chunks; row t routes over chunks c < floor(t/C);
  * the diagonal chunk is always attended, causally (keys j <= t), with log-prior 0;
  * g for a key in routed chunk c is the head-averaged block weight w_bar[c];
    sigma multiplies log g (sigma = 1 makes the bias exactly log w_bar);
  * a score exactly at the threshold gets weight 0 and mask bit 0.

A top-k router (route_row_topk) is here for comparison only: it is not the method.

Parity pins for this file live in tests/test_oracle_*.py.  The scale choices
(1/sqrt(D) in Stages 0 and 2, gamma/sqrt(D) in Stage 1), the head_cls shape [Hkv, D],
the diagonal branch and sigma are readings with no printed example: "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

CHUNK = 64


# ---------------------------------------------------------------------------------------
# Elementary transforms
# ---------------------------------------------------------------------------------------

def softmax(x: np.ndarray, axis: int = -1) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def _exact_tau_on_support(y: np.ndarray, in_s: np.ndarray, alpha: float) -> np.ndarray:
    """Closed-form threshold for a known support S (alpha in {1.5, 2}).

    alpha = 2  :  sum_S (y - tau) = 1            ->  tau = (sum_S y - 1) / |S|
    alpha = 1.5:  sum_S (y - tau)^2 = 1 (root below the support mean)
                  ->  tau = mean_S - sqrt(1/|S| - var_S)
    Rows whose support gives no real root return nan."""
    n = in_s.sum(axis=-1).astype(np.float64)
    n_safe = np.maximum(n, 1.0)
    ys = np.where(in_s, y, 0.0)
    mean = ys.sum(axis=-1) / n_safe
    if alpha == 2.0:
        return (ys.sum(axis=-1) - 1.0) / n_safe
    dev = np.where(in_s, y - mean[..., None], 0.0)
    var = (dev * dev).sum(axis=-1) / n_safe
    disc = 1.0 / n_safe - var
    with np.errstate(invalid="ignore"):
        return np.where(disc >= 0.0, mean - np.sqrt(np.maximum(disc, 0.0)), np.nan)


def entmax(x: np.ndarray, alpha: float, return_tau: bool = False):
    """alpha-entmax along the last axis by bisection on the threshold.

    Steps: y = (alpha - 1) x; tau lies in [max y - 1, max y - n^(1 - alpha)] (the top
    element alone gives f >= 0 at the left end, n equal elements bound the right end);
    bisect f(tau) = sum [y - tau]_+^(1/(alpha-1)) - 1 until the bracket is below
    2^-50 max(1, |max y|); for alpha in {1.5, 2} finish with the closed form on the
    support and keep it if it is self-consistent; p = [y - tau]_+^(1/(alpha-1)),
    normalised to sum 1.

    Returns p (and, if asked, tau and y) with the same leading shape as x."""
    if not (alpha > 1.0) or not math.isfinite(alpha):
        raise ValueError("alpha must be finite and > 1")
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n == 0:
        raise ValueError("entmax of an empty vector")
    y = (alpha - 1.0) * x
    inv = 1.0 / (alpha - 1.0)
    ymax = y.max(axis=-1)
    lo = ymax - 1.0
    hi = ymax - float(n) ** (1.0 - alpha)
    tol = 2.0 ** -50 * np.maximum(1.0, np.abs(ymax))

    def f(tau):
        return (np.maximum(y - tau[..., None], 0.0) ** inv).sum(axis=-1) - 1.0

    for _ in range(400):
        if np.all(hi - lo <= tol):
            break
        mid = 0.5 * (lo + hi)
        fm = f(mid)
        lo = np.where(fm >= 0.0, mid, lo)
        hi = np.where(fm >= 0.0, hi, mid)
    tau = 0.5 * (lo + hi)

    if alpha in (1.5, 2.0):
        # the true support is {y > tau*}; with tau* in [lo, hi] it is one of these two
        for cand in (y > lo[..., None], y > hi[..., None]):
            t_c = _exact_tau_on_support(y, cand, alpha)
            inside = np.where(cand, y, np.inf).min(axis=-1)
            outside = np.where(cand, -np.inf, y).max(axis=-1)
            ok = np.isfinite(t_c) & (inside > t_c) & (outside <= t_c) & cand.any(axis=-1)
            tau = np.where(ok, t_c, tau)

    p = np.maximum(y - tau[..., None], 0.0) ** inv
    p = p / p.sum(axis=-1, keepdims=True)
    if return_tau:
        return p, tau, y
    return p


def sparsemax_sorted(x: np.ndarray) -> np.ndarray:
    """Sparsemax by the sort-based closed form of Martins and Astudillo (2016), 1-D."""
    z = np.asarray(x, dtype=np.float64)
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, z.size + 1)
    support = 1.0 + k * zs > cs
    kz = k[support][-1]
    tau = (cs[kz - 1] - 1.0) / kz
    return np.maximum(z - tau, 0.0)


def entmax15_sorted(x: np.ndarray) -> np.ndarray:
    """1.5-entmax by exhaustive search over sorted supports, 1-D (Peters et al. 2019).

    For each k the candidate threshold solves sum_{j<=k} (z_(j) - tau)^2 = 1 on the k
    largest z = x/2; the answer is the k whose threshold keeps exactly those k above it."""
    z = np.asarray(x, dtype=np.float64) / 2.0
    zs = np.sort(z)[::-1]
    n = z.size
    tau = None
    for k in range(1, n + 1):
        top = zs[:k]
        mean = top.mean()
        var = ((top - mean) ** 2).mean()
        disc = 1.0 / k - var
        if disc < 0.0:
            continue
        t = mean - math.sqrt(disc)
        if zs[k - 1] > t and (k == n or zs[k] <= t):
            tau = t
            break
    if tau is None:
        raise RuntimeError("no consistent support found")
    return np.maximum(z - tau, 0.0) ** 2


def entmax_sorted_general(x: np.ndarray, alpha: float) -> np.ndarray:
    """alpha-entmax for any alpha > 1 by search over sorted supports, 1-D.

    For support size k the threshold solves  sum_{j<=k} (y_(j) - tau)^(1/(alpha-1)) = 1
    for tau in [y_(k+1), y_(k)); that equation is monotone there, so a per-interval
    bisection settles it.  Independent of the global bisection in `entmax`."""
    y = (alpha - 1.0) * np.asarray(x, dtype=np.float64)
    ys = np.sort(y)[::-1]
    n = y.size
    inv = 1.0 / (alpha - 1.0)
    for k in range(1, n + 1):
        top = ys[:k]
        hi_t = ys[k - 1]
        lo_t = ys[k] if k < n else ys[k - 1] - 2.0
        g = lambda t: (np.maximum(top - t, 0.0) ** inv).sum() - 1.0
        # g equals the full equation on [y_(k+1), y_(k)); the first k with g(y_(k+1)) >= 0
        # brackets the root there (g(y_(k)) < 0 held for the previous k).
        if g(lo_t) >= 0.0:
            a, b = lo_t, hi_t
            for _ in range(200):
                m = 0.5 * (a + b)
                if g(m) >= 0.0:
                    a = m
                else:
                    b = m
            tau = 0.5 * (a + b)
            return np.maximum(y - tau, 0.0) ** inv / (np.maximum(y - tau, 0.0) ** inv).sum()
    raise RuntimeError("unreachable: some support size always brackets the root")


def tsallis_objective(p: np.ndarray, x: np.ndarray, alpha: float) -> float:
    """p.x + sum_j (p_j - p_j^alpha) / (alpha (alpha - 1))."""
    p = np.asarray(p, dtype=np.float64)
    return float(p @ x + (p - p ** alpha).sum() / (alpha * (alpha - 1.0)))


def prior_softmax(z: np.ndarray, g: np.ndarray) -> np.ndarray:
    """argmax_p z.p - KL(p || g) = g exp(z) / sum g exp(z); zero where g = 0."""
    z = np.asarray(z, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return softmax(z + np.log(g))


# ---------------------------------------------------------------------------------------
# Stage 0
# ---------------------------------------------------------------------------------------

def chunk_summaries(k: np.ndarray, head_cls: np.ndarray, scale: float,
                    chunk: int = CHUNK) -> np.ndarray:
    """k [B, Hkv, T, D], head_cls [Hkv, D]  ->  summaries [B, Hkv, floor(T/C), D].

    For each complete chunk: a_j = scale <q_bar, k_j>, pi = softmax(a), k_bar = sum pi_j k_j.
    """
    k = np.asarray(k, dtype=np.float64)
    hc = np.asarray(head_cls, dtype=np.float64)
    B, H, T, D = k.shape
    nf = T // chunk
    kc = k[:, :, : nf * chunk].reshape(B, H, nf, chunk, D)
    a = scale * np.einsum("bhncd,hd->bhnc", kc, hc)
    pi = softmax(a, axis=-1)
    return np.einsum("bhnc,bhncd->bhnd", pi, kc)


# ---------------------------------------------------------------------------------------
# Stage 1: routing of one row (all G heads of one KV head)
# ---------------------------------------------------------------------------------------

def diagonal_summary(k_head: np.ndarray, head_cls_vec: np.ndarray, t: int, scale: float,
                     chunk: int = CHUNK) -> np.ndarray:
    """Summary of the query's own, partial chunk: Stage 0's formula over its keys up to t
    (keys i_t C .. t of one KV head; k_head [>= t+1, D])."""
    it = t // chunk
    kc = np.asarray(k_head[it * chunk: t + 1], np.float64)
    a = scale * (kc @ np.asarray(head_cls_vec, np.float64))
    return softmax(a) @ kc


def route_row(q_group: np.ndarray, summ: np.ndarray, t: int, *, alpha: float,
              gamma: float, scale: float, chunk: int = CHUNK,
              diag: Optional[np.ndarray] = None):
    """q_group [G, D]: the G query heads of one KV head at row t; summ [>= t//C, D].

    diag (estimate_diagonal): the summary of the query's own chunk, which then joins the
    alpha-entmax normalisation as one more entry; only the routed chunks' weights are
    returned (the own chunk stays attended with log-prior 0).
    Returns (w_bar [i_t], group_margin [i_t], p [G, i_t]) where i_t = t // C,
    group_margin_c = max_h (y_{h,c} - tau_h).  Empty arrays when i_t = 0."""
    it = t // chunk
    G = q_group.shape[0]
    if it == 0:
        return np.zeros(0), np.zeros(0), np.zeros((G, 0))
    keys = np.asarray(summ[:it], np.float64)
    if diag is not None:
        keys = np.concatenate([keys, np.asarray(diag, np.float64)[None, :]], axis=0)
    x = gamma * scale * (np.asarray(q_group, np.float64) @ keys.T)
    p, tau, y = entmax(x, alpha, return_tau=True)
    p, y = p[:, :it], y[:, :it]
    w_bar = p.mean(axis=0)
    margin = (y - tau[:, None]).max(axis=0)
    return w_bar, margin, p


def route_row_topk(q_group: np.ndarray, summ: np.ndarray, t: int, *, k: int, gamma: float,
                   scale: float, chunk: int = CHUNK):
    """Top-k routing, the comparison router (not the method's entmax): the group score of
    chunk c is the mean over the G heads of gamma * scale * <q_h, summ_c>; the chunks whose
    group score is at least the k-th largest are selected (every routed chunk when
    i_t <= k), each with weight 1, i.e. no prior.

    Returns (w_bar [i_t] in {0, 1}, margin [i_t] = group score - k-th largest)."""
    it = t // chunk
    if it == 0:
        return np.zeros(0), np.zeros(0)
    x = gamma * scale * (np.asarray(q_group, np.float64) @ np.asarray(summ[:it], np.float64).T)
    z = x.mean(axis=0)
    if it <= k:
        return np.ones(it), np.full(it, np.inf)
    kth = np.sort(z)[it - k]
    return (z >= kth).astype(np.float64), z - kth


# ---------------------------------------------------------------------------------------
# Stage 2: attention of one query row over the diagonal chunk and the routed chunks
# ---------------------------------------------------------------------------------------

def attend_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, t: int, w_bar: np.ndarray,
               *, scale: float, sigma: float = 1.0, chunk: int = CHUNK) -> np.ndarray:
    """q [D] one head at row t; k, v [>= t+1, D] of its KV head; w_bar [t // C].

    Keys of routed chunks with w_bar > 0 get bias sigma * log w_bar; keys of the own
    chunk up to t get bias 0; everything else is excluded.  Returns o [D]."""
    it = t // chunk
    idx, bias = [], []
    for c in range(it):
        if w_bar[c] > 0.0:
            idx.extend(range(c * chunk, (c + 1) * chunk))
            bias.extend([sigma * math.log(w_bar[c])] * chunk)
    idx.extend(range(it * chunk, t + 1))
    bias.extend([0.0] * (t + 1 - it * chunk))
    idx = np.asarray(idx)
    kk = np.asarray(k[idx], np.float64)
    vv = np.asarray(v[idx], np.float64)
    logits = scale * (kk @ np.asarray(q, np.float64)) + np.asarray(bias)
    return softmax(logits) @ vv


# ---------------------------------------------------------------------------------------
# Whole prefill (block walk, row by row)
# ---------------------------------------------------------------------------------------

def prefill(q, k, v, head_cls, *, alpha: float = 1.5, gamma: float = 1.0,
            scale: Optional[float] = None, sigma: float = 1.0, chunk: int = CHUNK,
            rows: Optional[Sequence[int]] = None, summaries: Optional[np.ndarray] = None,
            topk: int = 0, estimate_diagonal: bool = False) -> Dict[str, np.ndarray]:
    """Causal prefill.  q [B, Hq, T, D]; k, v [B, Hkv, T, D]; head_cls [Hkv, D].

    kv(h) = h // (Hq / Hkv).  `rows` restricts the rows computed (all by default).
    topk > 0 routes with `route_row_topk` instead of entmax (margin: score - k-th score).
    estimate_diagonal: the own chunk's partial summary joins each row's entmax.
    Returns out [B, Hq, R, D], w_bar [B, Hkv, R, n_c], margin [B, Hkv, R, n_c]
    (nan where c >= t // C), mask [B, Hkv, R, n_c] (w_bar > 0), rows [R], summaries."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nc = -(-T // chunk)
    rows = np.arange(T) if rows is None else np.asarray(rows)
    if summaries is None:
        summaries = chunk_summaries(k, head_cls, scale, chunk)
    R = rows.size
    out = np.zeros((B, Hq, R, D))
    w_bar = np.zeros((B, Hkv, R, nc))
    margin = np.full((B, Hkv, R, nc), np.nan)
    for b in range(B):
        for kvh in range(Hkv):
            kk = np.asarray(k[b, kvh], np.float64)
            vv = np.asarray(v[b, kvh], np.float64)
            for r, t in enumerate(rows):
                t = int(t)
                qg = np.asarray(q[b, kvh * G:(kvh + 1) * G, t], np.float64)
                if topk > 0:
                    wb, mg = route_row_topk(qg, summaries[b, kvh], t, k=topk, gamma=gamma,
                                            scale=scale, chunk=chunk)
                else:
                    dg = (diagonal_summary(kk, head_cls[kvh], t, scale, chunk)
                          if estimate_diagonal else None)
                    wb, mg, _ = route_row(qg, summaries[b, kvh], t, alpha=alpha, gamma=gamma,
                                          scale=scale, chunk=chunk, diag=dg)
                it = t // chunk
                w_bar[b, kvh, r, :it] = wb
                margin[b, kvh, r, :it] = mg
                for g in range(G):
                    out[b, kvh * G + g, r] = attend_row(qg[g], kk, vv, t, wb, scale=scale,
                                                        sigma=sigma, chunk=chunk)
    return {"out": out, "w_bar": w_bar, "margin": margin, "mask": w_bar > 0.0,
            "rows": rows, "summaries": summaries}


# ---------------------------------------------------------------------------------------
# Independent formulation: explicit T x T bias matrix (tiny T only)
# ---------------------------------------------------------------------------------------

def prefill_dense_formulation(q, k, v, head_cls, *, alpha: float, gamma: float = 1.0,
                              scale: Optional[float] = None, sigma: float = 1.0,
                              chunk: int = CHUNK, estimate_diagonal: bool = False) -> np.ndarray:
    """Same result as `prefill(...)["out"]`, written as one masked softmax per head.

    Summaries by explicit loops, routing weights by the sorted-support entmax, and the
    Stage 2 prior as a T x T additive matrix with -inf for excluded keys."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    hc = np.asarray(head_cls, np.float64)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nf = T // chunk
    out = np.zeros_like(q)
    for b in range(B):
        for kvh in range(Hkv):
            summ = np.zeros((nf, D))
            for c in range(nf):
                a = np.array([scale * float(hc[kvh] @ k[b, kvh, c * chunk + j])
                              for j in range(chunk)])
                e = np.exp(a - a.max())
                summ[c] = sum((e[j] / e.sum()) * k[b, kvh, c * chunk + j] for j in range(chunk))
            bias = np.full((T, T), -np.inf)
            for t in range(T):
                it = t // chunk
                if it > 0:
                    keys = summ[:it]
                    if estimate_diagonal:             # the own chunk's keys up to t, looped
                        n = t + 1 - it * chunk
                        a = np.array([scale * float(hc[kvh] @ k[b, kvh, it * chunk + j])
                                      for j in range(n)])
                        e = np.exp(a - a.max())
                        dg = sum((e[j] / e.sum()) * k[b, kvh, it * chunk + j] for j in range(n))
                        keys = np.vstack([keys, dg])
                    wsum = np.zeros(it)
                    for g in range(G):
                        x = gamma * scale * (keys @ q[b, kvh * G + g, t])
                        if alpha == 2.0:
                            wsum += sparsemax_sorted(x)[:it]
                        elif alpha == 1.5:
                            wsum += entmax15_sorted(x)[:it]
                        else:
                            wsum += entmax_sorted_general(x, alpha)[:it]
                    wbar = wsum / G
                    for c in range(it):
                        if wbar[c] > 0.0:
                            bias[t, c * chunk:(c + 1) * chunk] = sigma * math.log(wbar[c])
                bias[t, it * chunk:t + 1] = 0.0
            for g in range(G):
                h = kvh * G + g
                logits = scale * q[b, h] @ k[b, kvh].T + bias
                out[b, h] = softmax(logits, axis=-1) @ v[b, kvh]
    return out


def causal_attention(q, k, v, scale: Optional[float] = None) -> np.ndarray:
    """Textbook causal softmax attention, one head: q, k, v [T, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = scale * q @ k.T
    s[np.triu_indices(T, 1)] = -np.inf
    return softmax(s, axis=-1) @ v


# ---------------------------------------------------------------------------------------
# Decode: one new query per sequence against a cache and a summary cache
# ---------------------------------------------------------------------------------------

def decode_step(q_step, k_cache, v_cache, seq_lens, summary_cache, *, alpha: float = 1.5,
                gamma: float = 1.0, scale: Optional[float] = None, sigma: float = 1.0,
                chunk: int = CHUNK, head_cls: Optional[np.ndarray] = None,
                estimate_diagonal: bool = False) -> Dict[str, np.ndarray]:
    """q_step [B, Hq, D]; caches [B, Hkv, T_max, D]; seq_lens [B] (tokens in the cache,
    the current one included); summary_cache [B, Hkv, >= n, D] holding at least the
    summaries of every complete chunk before the current one.

    The query sits at t = seq_len - 1; it routes over chunks c < t // C (their summaries
    were frozen when each chunk filled) and attends causally inside its own chunk."""
    B, Hq, D = q_step.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    T_max = k_cache.shape[2]
    nc = -(-T_max // chunk)
    out = np.zeros((B, Hq, D))
    w_bar = np.zeros((B, Hkv, nc))
    margin = np.full((B, Hkv, nc), np.nan)
    for b in range(B):
        t = int(seq_lens[b]) - 1
        for kvh in range(Hkv):
            qg = np.asarray(q_step[b, kvh * G:(kvh + 1) * G], np.float64)
            dg = (diagonal_summary(k_cache[b, kvh], head_cls[kvh], t, scale, chunk)
                  if estimate_diagonal else None)
            wb, mg, _ = route_row(qg, summary_cache[b, kvh], t, alpha=alpha, gamma=gamma,
                                  scale=scale, chunk=chunk, diag=dg)
            it = t // chunk
            w_bar[b, kvh, :it] = wb
            margin[b, kvh, :it] = mg
            kk = np.asarray(k_cache[b, kvh, : t + 1], np.float64)
            vv = np.asarray(v_cache[b, kvh, : t + 1], np.float64)
            for g in range(G):
                out[b, kvh * G + g] = attend_row(qg[g], kk, vv, t, wb, scale=scale,
                                                 sigma=sigma, chunk=chunk)
    return {"out": out, "w_bar": w_bar, "margin": margin, "mask": w_bar > 0.0}


# ---------------------------------------------------------------------------------------
# Sparsity accounting
# ---------------------------------------------------------------------------------------

def zero_fraction(w_bar: np.ndarray, rows: np.ndarray, chunk: int = CHUNK) -> float:
    """Fraction of routed (row, kv head, chunk c < t // C) pairs with w_bar == 0.
    The diagonal chunk is not counted."""
    tot = 0
    zero = 0
    for r, t in enumerate(np.asarray(rows)):
        it = int(t) // chunk
        if it == 0:
            continue
        seg = w_bar[..., r, :it]
        tot += seg.size
        zero += int((seg == 0.0).sum())
    return zero / tot if tot else 0.0
