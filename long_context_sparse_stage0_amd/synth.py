"""Seeded synthetic inputs for the DashAttention forward pass.

This module is shared by the CPU oracle tests and by the GPU path's tests and benchmark.
It builds inputs only -- queries, keys, values and the per-KV-head classifier query -- and
holds none of the method's arithmetic.

Recipe (stated once here, repeated in the design notes):
  * K, V ~ N(0, 1) with shape [B, Hkv, T, D]; head_cls ~ N(0, 1) * head_cls_std, [Hkv, D].
  * Q is either i.i.d. N(0, 1), or "block-coherent": for every (b, kv head, 64-row query
    block) a direction mu ~ N(0, I_D) is shared by the G query heads of that kv head and
    the 64 rows of the block:  Q = (mu + j * eps) / sqrt(1 + j^2), eps ~ N(0, I_D).
    Each element is still marginally N(0, 1).
  * Needles: for every query block beta >= 1 of every (b, kv head), n_beta earlier chunks
    (uniform count in 1..32, or Poisson(lambda), clipped to beta) are drawn without
    replacement from [0, beta); their 64 keys are shifted by  A * u,  where u is the unit
    vector along the mean query of that block (over its rows and the group's heads).
    Shifts accumulate in float64 and the keys are rounded once to the storage dtype.
  * Decode: the "query blocks" are the blocks of 64 consecutive decode steps; their
    needles land in the chunks of the initial cache.
  * bf16 rounding is round-to-nearest-even.  Every draw comes from its own PCG64 stream,
    keyed by (seed, tensor id, b, kv head), so generation order does not matter.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict

import numpy as np

from .workloads import CHUNK, Workload

_Q, _K, _V, _HC, _NEEDLE = 1, 2, 3, 4, 5


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float32/float64 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF) + lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x_bf16_in_f32: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x_bf16_in_f32, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _queries(w: Workload, b: int, kvh: int, n_rows: int) -> np.ndarray:
    """[G, n_rows, D] queries of the G heads sharing kv head `kvh`."""
    rng = _rng(w.seed, _Q, b, kvh)
    G, D = w.G, w.D
    if w.q_mode == "iid":
        q = rng.standard_normal((G, n_rows, D), dtype=np.float32)
    else:
        nblk = -(-n_rows // CHUNK)
        mu = rng.standard_normal((nblk, D)).astype(np.float32)
        q = rng.standard_normal((G, n_rows, D), dtype=np.float32)
        q *= np.float32(w.coherence_j)
        q += np.repeat(mu, CHUNK, axis=0)[:n_rows][None]
        q *= np.float32(1.0 / math.sqrt(1.0 + w.coherence_j ** 2))
    return _store(q, w.dtype)


def _needle_shifts(w: Workload, b: int, kvh: int, q_group: np.ndarray,
                   n_chunks: int, first_block: int, block_limit) -> np.ndarray:
    """float64 [n_chunks, D] accumulated needle shifts for one (b, kv head).

    q_group: [G, R, D] queries; query block i covers rows [64 i, 64 i + 64) of it and
    plants needles into chunks [0, block_limit(i)).
    """
    shift = np.zeros((n_chunks, w.D))
    if w.needle_count == "none" or w.needle_amp == 0.0:
        return shift
    rng = _rng(w.seed, _NEEDLE, b, kvh)
    R = q_group.shape[1]
    nqb = -(-R // CHUNK)
    for i in range(first_block, nqb):
        lim = block_limit(i)
        if lim <= 0:
            continue
        if w.needle_count == "uniform32":
            n = int(rng.integers(1, 33))
        else:
            n = int(rng.poisson(w.needle_lambda))
        n = min(n, lim)
        if n == 0:
            continue
        chunks = rng.choice(lim, size=n, replace=False)
        m = q_group[:, i * CHUNK:(i + 1) * CHUNK, :].astype(np.float64).mean(axis=(0, 1))
        nrm = np.linalg.norm(m)
        if nrm == 0.0:
            continue
        shift[chunks] += w.needle_amp * (m / nrm)
    return shift


def _keys(w: Workload, b: int, kvh: int, n_rows: int, shift: np.ndarray) -> np.ndarray:
    rng = _rng(w.seed, _K, b, kvh)
    k = rng.standard_normal((n_rows, w.D))
    nfull = min(shift.shape[0], n_rows // CHUNK)
    k[: nfull * CHUNK] += np.repeat(shift[:nfull], CHUNK, axis=0)
    return _store(k, w.dtype)


def _values(w: Workload, b: int, kvh: int, n_rows: int) -> np.ndarray:
    rng = _rng(w.seed, _V, b, kvh)
    return _store(rng.standard_normal((n_rows, w.D), dtype=np.float32), w.dtype)


def head_cls(w: Workload) -> np.ndarray:
    rng = _rng(w.seed, _HC)
    return _store(rng.standard_normal((w.Hkv, w.D)) * w.head_cls_std, w.dtype)


def _parallel(fn, items, workers):
    if workers <= 1 or len(items) <= 1:
        return [fn(*it) for it in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda it: fn(*it), items))


def prefill_inputs(w: Workload, workers: int = 8) -> Dict[str, np.ndarray]:
    """q [B,Hq,T,D], k, v [B,Hkv,T,D], head_cls [Hkv,D] (float32 arrays holding values
    representable in the workload dtype)."""
    assert w.kind == "prefill"
    B, Hq, Hkv, T, D, G = w.B, w.Hq, w.Hkv, w.T, w.D, w.G
    q = np.empty((B, Hq, T, D), np.float32)
    k = np.empty((B, Hkv, T, D), np.float32)
    v = np.empty((B, Hkv, T, D), np.float32)

    def one(b, h):
        qg = _queries(w, b, h, T)
        q[b, h * G:(h + 1) * G] = qg
        shift = _needle_shifts(w, b, h, qg, T // CHUNK, 1, lambda i: i)
        k[b, h] = _keys(w, b, h, T, shift)
        v[b, h] = _values(w, b, h, T)

    _parallel(one, [(b, h) for b in range(B) for h in range(Hkv)], workers)
    return {"q": q, "k": k, "v": v, "head_cls": head_cls(w)}


def decode_inputs(w: Workload, workers: int = 8) -> Dict[str, np.ndarray]:
    """k_cache, v_cache [B,Hkv,T+steps,D] holding the initial T tokens followed by the keys
    and values of the `steps` new tokens; q_steps [steps,B,Hq,D]; head_cls [Hkv,D]."""
    assert w.kind == "decode"
    B, Hq, Hkv, D, G, S = w.B, w.Hq, w.Hkv, w.D, w.G, w.steps
    TT = w.T + S
    k = np.empty((B, Hkv, TT, D), np.float32)
    v = np.empty((B, Hkv, TT, D), np.float32)
    qs = np.empty((S, B, Hq, D), np.float32)
    n_init_chunks = w.T // CHUNK

    def one(b, h):
        qg = _queries(w, b, h, S)                     # [G, S, D], blocks of 64 steps
        qs[:, b, h * G:(h + 1) * G] = np.transpose(qg, (1, 0, 2))
        shift = _needle_shifts(w, b, h, qg, TT // CHUNK, 0, lambda i: n_init_chunks)
        k[b, h] = _keys(w, b, h, TT, shift)
        v[b, h] = _values(w, b, h, TT)

    _parallel(one, [(b, h) for b in range(B) for h in range(Hkv)], workers)
    return {"q_steps": qs, "k_cache": k, "v_cache": v, "head_cls": head_cls(w)}


def chunk_valued_prefill(T: int, D: int, G: int, dist: str, amp: float, seed: int,
                         dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """Prefill inputs whose chunks carry prescribed values (B = 1, one kv head, G heads).

    Every key of chunk c equals one vector whose first coordinate is u_c, drawn from `dist`,
    and whose other coordinates are N(0, 1); head_cls is zero; every query of head h is
    amp * (1 + h / 32) along the first axis.  So the chunk-level logits of a row are
    u_c scaled by the query's length, with the shape of `dist`:
      "uniform"        u ~ U(0, 1)
      "left_outliers"  u ~ N(0, 0.05), with a tenth of the chunks at N(-0.8, 0.01)
      "exp_left"       u = -E, E ~ Exp(mean 0.1)
    V ~ N(0, 1).  Returns q [1,G,T,D], k, v [1,1,T,D], head_cls [1,D] as float32 arrays
    holding values representable in `dtype`."""
    nc = -(-T // CHUNK)
    r = _rng(seed, 7001)
    if dist == "uniform":
        u = r.uniform(0.0, 1.0, nc)
    elif dist == "left_outliers":
        u = r.normal(0.0, 0.05, nc)
        low = r.random(nc) < 0.1
        u[low] = r.normal(-0.8, 0.01, int(low.sum()))
    elif dist == "exp_left":
        u = -r.exponential(0.1, nc)
    else:
        raise ValueError(f"unknown distribution {dist}")
    kc = _rng(seed, 7002).standard_normal((nc, D))
    kc[:, 0] = u
    k = np.repeat(kc, CHUNK, axis=0)[:T][None, None]
    v = _rng(seed, 7003).standard_normal((1, 1, T, D))
    q = np.zeros((1, G, T, D))
    for h in range(G):
        q[0, h, :, 0] = amp * (1.0 + h / 32.0)
    return {"q": _store(q, dtype), "k": _store(k, dtype), "v": _store(v, dtype),
            "head_cls": np.zeros((1, D), np.float32)}
