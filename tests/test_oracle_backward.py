"""Pins of the float64 backward oracle (oracle/dash_oracle_backward.py) against what the
mathematics fixes, independently of its own formulas:

  * the entmax Jacobian-vector product equals central finite differences of the forward
    entmax, equals the sparsemax Jacobian's closed form at alpha = 2 (Martins and
    Astudillo 2016), and tends to the softmax Jacobian as alpha -> 1;
  * the whole backward equals torch autograd (float64, CPU) through a separately written
    forward -- summaries by softmax pooling, entmax by the sorted-support closed forms for
    alpha in {1.5, 2}, a dense T x T biased attention -- to 1e-9;
  * the whole backward equals central finite differences of the oracle's forward loss on
    tiny inputs (alpha = 1.25, the general case, and 1.5), skipping perturbations that move
    a routing support;
  * special cases: sigma = 0 cuts the routing gradient (d head_cls = 0 exactly).
"""
import math

import numpy as np
import pytest

from oracle import dash_oracle as F
from oracle import dash_oracle_backward as BW


def _margins_ok(x, alpha, gap=1e-3):
    p, tau, y = F.entmax(x, alpha, return_tau=True)
    return np.all(np.abs(y - tau[..., None]) > gap)


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0, 3.0])
def test_entmax_backward_matches_finite_differences(alpha):
    rng = np.random.default_rng(int(alpha * 100))
    n = 30
    for trial in range(20):
        x = rng.normal(size=n) * 2.0
        if not _margins_ok(x, alpha):
            continue
        dp = rng.normal(size=n)
        p = F.entmax(x, alpha)
        eps = 1e-6
        J = np.zeros((n, n))
        for i in range(n):
            e = np.zeros(n)
            e[i] = eps
            J[:, i] = (F.entmax(x + e, alpha) - F.entmax(x - e, alpha)) / (2 * eps)
        np.testing.assert_allclose(BW.entmax_backward(p, dp, alpha), J.T @ dp, atol=2e-7)


def test_entmax_backward_sparsemax_closed_form():
    """alpha = 2: the Jacobian is diag(1_S) - 1_S 1_S^T / |S| (sparsemax)."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        x = rng.normal(size=40)
        p = F.sparsemax_sorted(x)
        S = (p > 0).astype(np.float64)
        J = np.diag(S) - np.outer(S, S) / S.sum()
        dp = rng.normal(size=40)
        np.testing.assert_allclose(BW.entmax_backward(p, dp, 2.0), J @ dp, atol=1e-13)


def test_entmax_backward_tends_to_softmax_jacobian():
    """As alpha -> 1, p^(2 - alpha) -> p, so the Jacobian tends to diag(p) - p p^T."""
    rng = np.random.default_rng(8)
    x = rng.normal(size=25) * 0.5
    dp = rng.normal(size=25)
    sm = F.softmax(x)
    ref = sm * dp - sm * (sm @ dp)
    errs = []
    for eps in (1e-2, 1e-3):
        p = F.entmax(x, 1.0 + eps)
        errs.append(np.abs(BW.entmax_backward(p, dp, 1.0 + eps) - ref).max())
    assert errs[1] < errs[0] and errs[1] < 5e-3


# ------------------------------------------------------------------ autograd pin

torch = pytest.importorskip("torch")


def _entmax_sorted_torch(x, alpha):
    """alpha in {1.5, 2}: alpha-entmax along the last axis of a 1-D float64 tensor by the
    sorted-support closed forms; the support is chosen on detached values and the
    threshold is a differentiable function of the values on it."""
    z = (alpha - 1.0) * x
    zs, _ = torch.sort(z.detach(), descending=True)
    n = z.numel()
    for kk in range(1, n + 1):
        top = zs[:kk]
        if alpha == 2.0:
            t = (top.sum() - 1.0) / kk
        else:
            mean = top.mean()
            disc = 1.0 / kk - ((top - mean) ** 2).mean()
            if disc < 0:
                continue
            t = mean - math.sqrt(float(disc))
        if zs[kk - 1] > t and (kk == n or zs[kk] <= t):
            sup = z.detach() > t
            zsup = z[sup]
            if alpha == 2.0:
                tau = (zsup.sum() - 1.0) / kk
                return torch.clamp(z - tau, min=0.0)
            mean = zsup.mean()
            tau = mean - torch.sqrt(1.0 / kk - ((zsup - mean) ** 2).mean())
            return torch.clamp(z - tau, min=0.0) ** 2
    raise RuntimeError("no consistent support")


def _torch_forward(q, k, v, hc, *, alpha, gamma, sigma, scale):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    nf = T // 64
    kc = k[:, :, :nf * 64].reshape(B, Hkv, nf, 64, D)
    pi = torch.softmax(scale * torch.einsum("bhncd,hd->bhnc", kc, hc), dim=-1)
    summ = torch.einsum("bhnc,bhncd->bhnd", pi, kc)
    outs = []
    for b in range(B):
        for kvh in range(Hkv):
            bias_rows = []
            for t in range(T):
                it = t // 64
                row = torch.full((T,), -math.inf, dtype=torch.float64)
                if it > 0:
                    x = gamma * scale * (q[b, kvh * G:(kvh + 1) * G, t] @ summ[b, kvh, :it].T)
                    wbar = torch.stack([_entmax_sorted_torch(x[g], alpha) for g in range(G)]).mean(0)
                    on = wbar.detach() > 0
                    lw = torch.where(on, torch.log(torch.where(on, wbar, torch.ones_like(wbar))),
                                     torch.full_like(wbar, -math.inf))
                    row = torch.cat([torch.repeat_interleave(sigma * lw, 64),
                                     torch.full((T - it * 64,), -math.inf, dtype=torch.float64)])
                diag = torch.zeros(T, dtype=torch.bool)
                diag[it * 64:t + 1] = True
                row = torch.where(diag, torch.zeros_like(row), row)
                bias_rows.append(row)
            bias = torch.stack(bias_rows)
            for g in range(G):
                h = kvh * G + g
                logits = scale * q[b, h] @ k[b, kvh].T + bias
                outs.append(torch.softmax(logits, dim=-1) @ v[b, kvh])
    return torch.stack(outs).reshape(B, Hq, T, D)


@pytest.mark.parametrize("alpha,G,sigma", [(1.5, 2, 1.0), (2.0, 2, 1.0), (1.5, 1, 0.5),
                                           (1.5, 4, 2.0)])
def test_backward_matches_autograd(alpha, G, sigma):
    rng = np.random.default_rng(300 + G + int(10 * alpha))
    B, Hkv, T, D = 1, 2, 200, 8
    Hq = G * Hkv
    q = rng.normal(size=(B, Hq, T, D))
    k = rng.normal(size=(B, Hkv, T, D))
    v = rng.normal(size=(B, Hkv, T, D))
    hc = rng.normal(size=(Hkv, D))
    # sharper routing logits so that several chunks fall outside the support
    q *= 3.0
    dout = rng.normal(size=(B, Hq, T, D))
    scale = 1.0 / math.sqrt(D)
    ref = BW.prefill_backward(q, k, v, hc, dout, alpha=alpha, sigma=sigma)
    tq, tk, tv, th = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                      for a in (q, k, v, hc))
    out = _torch_forward(tq, tk, tv, th, alpha=alpha, gamma=1.0, sigma=sigma, scale=scale)
    np.testing.assert_allclose(out.detach().numpy(),
                               F.prefill(q, k, v, hc, alpha=alpha, sigma=sigma)["out"],
                               atol=1e-12)
    (out * torch.tensor(dout)).sum().backward()
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv), ("dhead_cls", th)):
        np.testing.assert_allclose(ref[name], t.grad.numpy(), atol=1e-9, rtol=1e-9,
                                   err_msg=name)
    # the routing gradient really reaches Stage 0
    assert np.abs(ref["dhead_cls"]).max() > 1e-6


# ------------------------------------------------------------------ finite differences

@pytest.mark.parametrize("alpha", [1.25, 1.5])
def test_backward_matches_finite_differences(alpha):
    rng = np.random.default_rng(400 + int(alpha * 100))
    B, Hkv, G, T, D = 1, 1, 2, 150, 4
    Hq = G * Hkv
    x = {"q": 2.0 * rng.normal(size=(B, Hq, T, D)), "k": rng.normal(size=(B, Hkv, T, D)),
         "v": rng.normal(size=(B, Hkv, T, D)), "head_cls": rng.normal(size=(Hkv, D))}
    dout = rng.normal(size=(B, Hq, T, D))
    ref = BW.prefill_backward(x["q"], x["k"], x["v"], x["head_cls"], dout, alpha=alpha)
    grads = {"q": ref["dq"], "k": ref["dk"], "v": ref["dv"], "head_cls": ref["dhead_cls"]}
    eps = 1e-5

    def run(xx):
        r = F.prefill(xx["q"], xx["k"], xx["v"], xx["head_cls"], alpha=alpha)
        return float((dout * r["out"]).sum()), r["mask"]

    _, mask0 = run(x)
    checked = 0
    for name in ("q", "k", "v", "head_cls"):
        n = x[name].size
        picks = range(n) if n <= 8 else rng.choice(n, size=12, replace=False)
        for i in picks:
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[name].flat[i] += eps
            xm[name].flat[i] -= eps
            lp, mp = run(xp)
            lm, mm = run(xm)
            if not (np.array_equal(mp, mask0) and np.array_equal(mm, mask0)):
                continue                      # the perturbation moves a routing support
            fd = (lp - lm) / (2 * eps)
            g = grads[name].flat[i]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(g)), (name, i, fd, g)
            checked += 1
    assert checked >= 30


def test_sigma_zero_cuts_routing_gradient():
    """With sigma = 0 the prior is uniform over the active chunks: nothing depends on the
    weights' values, so no gradient reaches Stage 1 or Stage 0."""
    rng = np.random.default_rng(9)
    q = rng.normal(size=(1, 2, 140, 8)) * 2
    k = rng.normal(size=(1, 1, 140, 8))
    v = rng.normal(size=(1, 1, 140, 8))
    hc = rng.normal(size=(1, 8))
    r = BW.prefill_backward(q, k, v, hc, rng.normal(size=q.shape), sigma=0.0)
    assert np.all(r["dhead_cls"] == 0.0) and np.all(r["dsumm"] == 0.0)
