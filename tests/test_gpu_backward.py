"""GPU parity of the backward pass (dash_prefill_train + dash_prefill_backward through the C
ABI) against the float64 backward oracle, on seeded inputs and a seeded dL/dout.

Tolerance (a reading: the pages fix none for gradients): the forward's output bar applied
to each gradient relative to its scale, max |g - ref| / max(1, max |ref|) <= 1e-4 for fp32
and 2e-2 for bf16.  A gradient is a sum over many rows of terms of the size the forward's
bar covers, so its error grows with its magnitude; dividing by max(1, max |ref|) keeps the
bar at the forward's where gradients are of order one.
"""
import numpy as np
import pytest

from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import PREFILL_1K_FP32, Workload
from oracle import dash_oracle as F
from oracle import dash_oracle_backward as BW
from tests.parity_util import say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

GRAD_TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_stage0_amd import dash as d
    d.load()
    return d


def _dout(shape, dtype, seed):
    g = np.random.default_rng(seed).normal(size=shape)
    return synth.round_bf16(g) if dtype == "bf16" else g.astype(np.float32)


def _check_grad(name, got, ref, dtype):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = float(np.abs(got - ref).max()) / max(1.0, float(np.abs(ref).max()))
    assert err <= GRAD_TOL[dtype], f"{name}: relative max error {err:.3e} > {GRAD_TOL[dtype]}"
    return err


def run_backward(dash, w, *, alpha=None, sigma=1.0, seed=1):
    alpha = w.alpha if alpha is None else alpha
    x = synth.prefill_inputs(w)
    dout = _dout(x["q"].shape, w.dtype, seed)
    say(f"[backward] {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} {w.dtype} "
        f"alpha={alpha} sigma={sigma}")
    q, k, v, hc = (to_dev(x[n], w.dtype) for n in ("q", "k", "v", "head_cls"))
    do = to_dev(dout, w.dtype)
    kw = dict(alpha=alpha, gamma=w.gamma, sigma=sigma, enable_gqa=w.enable_gqa)
    out, lse = dash.prefill_train(q, k, v, hc, **kw)
    plain = dash.prefill(q, k, v, hc, **kw)
    dq, dk, dv, dhc = dash.prefill_backward(q, k, v, hc, out, do, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain), "the training forward must equal dash_prefill"
    ref = BW.prefill_backward(x["q"], x["k"], x["v"], x["head_cls"], dout, alpha=alpha,
                              gamma=w.gamma, sigma=sigma)
    got = {n: g.float().cpu().numpy() for n, g in (("dq", dq), ("dk", dk), ("dv", dv), ("dhead_cls", dhc))}
    errs = {n: _check_grad(n, got[n], ref[n], w.dtype) for n in got}
    say("[backward]   " + "  ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    return x, ref, got


def test_backward_1k_fp32(dash):
    """The 1K fp32 workload (2 heads, D = 64, i.i.d. queries), every gradient."""
    run_backward(dash, PREFILL_1K_FP32)


@pytest.mark.parametrize("dtype,G,alpha,sigma,T,D", [
    ("bf16", 4, 1.5, 1.0, 700, 128),      # ragged tail
    ("bf16", 16, 1.5, 1.0, 400, 128),     # the 128K workload's head ratio
    ("bf16", 2, 1.25, 0.5, 333, 64),
    ("bf16", 1, 1.5, 1.0, 260, 64),       # no GQA (the 4-wave dQ instance)
    ("bf16", 8, 2.0, 1.0, 530, 128),
    ("fp32", 2, 1.25, 0.5, 300, 64),      # the general-alpha Jacobian
    ("fp32", 8, 1.5, 2.0, 450, 128),
])
def test_backward_small(dash, dtype, G, alpha, sigma, T, D):
    w = Workload(name=f"bwd_{dtype}_g{G}", kind="prefill", B=2 if dtype == "bf16" else 1,
                 Hq=2 * G, Hkv=2, T=T, D=D, dtype=dtype, alpha=alpha, seed=1200 + G,
                 needle_amp=1.0)
    _, ref, _ = run_backward(dash, w, sigma=sigma, seed=G)
    # the routing gradient is really exercised: it reaches Stage 0's classifier query
    assert np.abs(ref["dhead_cls"]).max() > 1e-3


def test_backward_routing_part_of_dq(dash):
    """Stage 1's part of dq, gamma scale dx K_bar with dx the entmax Jacobian applied to
    dL/dw_bar / G (the gradient that flows back through the router), is only a few percent
    of dq at gamma = sigma = 1, inside the bf16 bar of the whole dq.  Here gamma = 4 and
    sigma = 4 make it about a sixth of dq's norm, and dq's error is also measured against the
    norm of the oracle's Stage 1 part alone: the bf16 path's whole-dq error (about 3.5e-3 of
    |dq| in norm) is about 2% of that part, so a bar of 0.1 rejects a Stage 1 part that is
    wrong by more than a tenth of its norm."""
    G, T, D, gamma, sigma = 16, 400, 128, 4.0, 4.0
    w = Workload(name="bwd_route_part", kind="prefill", B=1, Hq=2 * G, Hkv=2, T=T, D=D,
                 dtype="bf16", gamma=gamma, seed=1600, needle_amp=1.0)
    x, ref, got = run_backward(dash, w, sigma=sigma, seed=16)
    scale = 1.0 / np.sqrt(D)
    summ = F.chunk_summaries(x["k"], x["head_cls"], scale)
    route = np.zeros_like(ref["dq"])
    for kvh in range(2):
        for t in range(64, T):
            qg = x["q"][0, G * kvh:G * (kvh + 1), t].astype(np.float64)
            _, _, p = F.route_row(qg, summ[0, kvh], t, alpha=1.5, gamma=gamma, scale=scale)
            dp = np.broadcast_to(ref["dw_bar"][0, kvh, t, :t // 64] / G, p.shape)
            dx = BW.entmax_backward(p, dp, 1.5)
            route[0, G * kvh:G * (kvh + 1), t] = gamma * scale * (dx @ summ[0, kvh, :t // 64])
    share = np.linalg.norm(route) / np.linalg.norm(ref["dq"])
    rel = np.linalg.norm(got["dq"] - ref["dq"]) / np.linalg.norm(route)
    say(f"[backward]   Stage 1 part {share:.3f} of |dq|; |dq error| / |Stage 1 part| {rel:.3e}")
    assert share > 0.1, "the Stage 1 part is too small here to be checked"
    assert rel <= 0.1, f"dq error {rel:.3e} of the Stage 1 part's norm"
    # dk's part through the summaries (Stage 0's softmax backward of dL/dK_bar), the same way
    dk_route, _ = BW.chunk_summaries_backward(x["k"], x["head_cls"], scale, ref["dsumm"])
    rel_k = np.linalg.norm(got["dk"] - ref["dk"]) / np.linalg.norm(dk_route)
    say(f"[backward]   |dk error| / |dk part through the summaries| {rel_k:.3e}")
    assert rel_k <= 0.1, f"dk error {rel_k:.3e} of its part through the summaries"


def test_backward_sparsemax_away_from_ties(dash):
    """alpha = 2 (sparsemax), whose Jacobian jumps where a chunk enters the support: on
    inputs where no routed chunk lies within 1e-4 of a threshold, GPU and oracle gradients
    agree."""
    w = Workload(name="bwd_a2", kind="prefill", B=1, Hq=4, Hkv=2, T=500, D=64, dtype="fp32",
                 alpha=2.0, seed=1300, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    r = F.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=2.0)
    m = r["margin"]
    assert np.nanmin(np.abs(m)) > 1e-4, "choose another seed: a chunk sits on a threshold"
    run_backward(dash, w)


def test_backward_tiny_sequences(dash):
    """Degenerate lengths: one chunk with no routing (every gradient from the diagonal
    branch; d head_cls = 0) and a partial second chunk."""
    for T in (50, 100):
        w = Workload(name=f"bwd_tiny{T}", kind="prefill", B=1, Hq=4, Hkv=2, T=T, D=64,
                     dtype="fp32", seed=1400 + T, needle_amp=1.0)
        _, ref, _ = run_backward(dash, w)
        # no routing (T = 50), or one routed chunk whose entmax weight is always 1
        assert np.abs(ref["dhead_cls"]).max() < 1e-12


def test_backward_bf16_dq_rows_and_dv_sum_at_8k(dash):
    """The MFMA backward at T = 8192 (32/2 heads): dq on sampled rows against the oracle's
    per-row backward (Stage 2 of each head, the GQA mean, the entmax Jacobian and the
    Stage 1 scores of that row), and a property of the whole dv: the attention weights of
    a row sum to one, so dv summed over the keys of a KV head equals dO summed over its
    rows and query heads."""
    from long_context_sparse_stage0_amd.workloads import CALIBRATED_AMP
    w = Workload(name="bwd_8k", kind="prefill", B=1, Hq=32, Hkv=2, T=8192, D=128,
                 dtype="bf16", seed=1500, needle_amp=CALIBRATED_AMP)
    x = synth.prefill_inputs(w)
    dout = _dout(x["q"].shape, "bf16", 15)
    say("[backward] 8K, 32/2 heads, sampled dq rows and the dv sum")
    q, k, v, hc = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "head_cls"))
    kw = dict(enable_gqa=True)
    out, lse = dash.prefill_train(q, k, v, hc, **kw)
    dq, dk, dv, dhc = dash.prefill_backward(q, k, v, hc, out, to_dev(dout, "bf16"), lse, **kw)
    torch.cuda.synchronize()
    g_dq = dq.float().cpu().numpy()
    g_dv = dv.float().cpu().numpy()
    assert np.isfinite(g_dq).all() and np.isfinite(g_dv).all()
    assert np.isfinite(dk.float().cpu().numpy()).all() and np.isfinite(dhc.cpu().numpy()).all()
    # dv property
    for kvh in range(2):
        lhs = g_dv[0, kvh].astype(np.float64).sum(axis=0)
        rhs = dout[0, 16 * kvh:16 * (kvh + 1)].astype(np.float64).sum(axis=(0, 1))
        err = np.abs(lhs - rhs).max() / max(1.0, np.abs(rhs).max())
        assert err <= 2e-2, f"dv sum, kv head {kvh}: {err:.3e}"
    # dq on sampled rows: the oracle's backward of one row
    scale = 1.0 / np.sqrt(w.D)
    summ = F.chunk_summaries(x["k"], x["head_cls"], scale)
    rows = [64, 127, 4095, 4096, 8191]
    for t in rows:
        for kvh in range(2):
            qg = x["q"][0, 16 * kvh:16 * (kvh + 1), t].astype(np.float64)
            wb, _, p = F.route_row(qg, summ[0, kvh], t, alpha=1.5, gamma=1.0, scale=scale)
            dwb = np.zeros(t // 64)
            ref = np.zeros((16, w.D))
            for g in range(16):
                dq_h, _, _, dwb_h = BW.attend_row_backward(
                    qg[g], x["k"][0, kvh], x["v"][0, kvh], t, wb,
                    dout[0, 16 * kvh + g, t], scale=scale)
                ref[g] = dq_h
                dwb += dwb_h
            if t // 64 > 0:
                dx = BW.entmax_backward(p, np.broadcast_to(dwb / 16, p.shape), 1.5)
                ref += scale * (dx @ summ[0, kvh, :t // 64])
            _check_grad(f"dq row {t} kv head {kvh}", g_dq[0, 16 * kvh:16 * (kvh + 1), t], ref,
                        "bf16")
