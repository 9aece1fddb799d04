"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on seeded
synthetic inputs, at sizes the oracle finishes in seconds, spanning several tiles and a
ragged tail."""
import math

import numpy as np
import pytest

from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import PREFILL_1K_FP32, Workload
from oracle import dash_oracle as O
from tests.parity_util import (compare_mask, compare_out, compare_weights, say, to_dev,
                               unpack_words)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_stage0_amd import dash as d
    d.load()
    return d


def run_prefill(dash, w: Workload, rows=None, alpha=None, sigma=1.0, topk=0,
                estimate_diagonal=False):
    alpha = w.alpha if alpha is None else alpha
    x = synth.prefill_inputs(w)
    say(f"[parity] prefill {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"{w.dtype} alpha={alpha} sigma={sigma} topk={topk} diag={estimate_diagonal}")
    q, k, v, hc = (to_dev(x[n], w.dtype) for n in ("q", "k", "v", "head_cls"))
    out, ab, bw, sm = dash.prefill(q, k, v, hc, alpha=alpha, gamma=w.gamma, sigma=sigma, topk=topk,
                                   estimate_diagonal=estimate_diagonal,
                                   enable_gqa=w.enable_gqa, return_active_blocks=True,
                                   return_block_weights=True, return_summaries=True)
    torch.cuda.synchronize()
    rows = np.arange(w.T) if rows is None else np.asarray(rows)
    ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=alpha, gamma=w.gamma,
                    sigma=sigma, rows=rows, topk=topk, estimate_diagonal=estimate_diagonal)
    nc = -(-w.T // 64)
    g_out = out.float().cpu().numpy()[:, :, rows]
    g_bits = unpack_words(ab.cpu().numpy(), nc)[:, :, rows]
    g_w = bw.cpu().numpy()[:, :, rows]
    g_s = sm.cpu().numpy()
    return dict(x=x, ref=ref, out=g_out, bits=g_bits, w=g_w, summ=g_s, rows=rows, nc=nc)


def check_prefill(r, w):
    nf = w.T // 64
    np.testing.assert_allclose(r["summ"][:, :, :nf], r["ref"]["summaries"], atol=2e-5, rtol=1e-5)
    e_out = compare_out(r["out"], r["ref"]["out"], w.dtype)
    e_w = compare_weights(r["w"], r["ref"]["w_bar"])
    amb = compare_mask(r["bits"], r["ref"]["mask"], r["ref"]["margin"], r["rows"])
    frac = O.zero_fraction(r["ref"]["w_bar"], r["rows"])
    say(f"[parity]   out err {e_out:.2e}  w err {e_w:.2e}  near-threshold flips {amb}  "
        f"zero-weight fraction {frac:.3f}")


def test_prefill_1k_fp32_full(dash):
    """The 1K fp32 workload, every row."""
    w = PREFILL_1K_FP32
    check_prefill(run_prefill(dash, w), w)


@pytest.mark.parametrize("G,alpha,T,D", [
    (4, 1.5, 1000, 128),     # ragged tail, GQA 4
    (16, 1.5, 700, 128),     # GQA 16 (the 128K workload's ratio)
    (1, 2.0, 520, 64),
    (2, 1.25, 450, 128),
    (8, 1.5, 333, 64),
])
def test_prefill_bf16_small(dash, G, alpha, T, D):
    w = Workload(name=f"small_g{G}", kind="prefill", B=2, Hq=2 * G, Hkv=2, T=T, D=D,
                 dtype="bf16", alpha=alpha, seed=900 + G, needle_amp=1.0)
    check_prefill(run_prefill(dash, w), w)


@pytest.mark.parametrize("dtype,sigma", [("bf16", 0.0), ("bf16", 0.5), ("bf16", 2.0),
                                         ("fp32", 0.0), ("fp32", 2.0)])
def test_prefill_prior_strength(dash, dtype, sigma):
    """Prior strength sigma != 1: routed keys get the bias sigma * log w_bar (0: a uniform
    prior over the active chunks)."""
    w = Workload(name=f"sigma_{dtype}", kind="prefill", B=1, Hq=8, Hkv=2, T=900, D=128,
                 dtype=dtype, seed=950, needle_amp=1.0)
    check_prefill(run_prefill(dash, w, sigma=sigma), w)


@pytest.mark.parametrize("dtype,G,alpha,T,D", [
    ("fp32", 4, 1.5, 1000, 128),     # ragged tail
    ("fp32", 1, 2.0, 520, 64),
    ("fp32", 16, 1.25, 700, 128),
    ("bf16", 16, 1.5, 1000, 128),    # k_diag_scores feeding the MFMA router
    ("bf16", 2, 2.0, 450, 64),
])
def test_prefill_estimate_diagonal(dash, dtype, G, alpha, T, D):
    """estimate_diagonal: the own chunk's partial summary joins each row's entmax; only the
    routed chunks' weights are kept."""
    w = Workload(name=f"diag_{dtype}_g{G}", kind="prefill", B=2 if dtype == "bf16" else 1,
                 Hq=2 * G, Hkv=2, T=T, D=D, dtype=dtype, alpha=alpha, seed=970 + G,
                 needle_amp=1.0)
    r = run_prefill(dash, w, estimate_diagonal=True)
    check_prefill(r, w)
    plain = run_prefill(dash, w, rows=r["rows"])
    assert np.abs(r["w"] - plain["w"]).max() > 1e-2    # the flag changes the weights


def test_decode_prior_strength(dash):
    """Decode with sigma = 2 equals the oracle's prefill row with the same sigma."""
    w = Workload(name="dec_sigma", kind="prefill", B=2, Hq=16, Hkv=2, T=1500, D=128,
                 dtype="bf16", seed=951, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say("[parity] decode sigma 2")
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    lens = [1500, 1000]
    nc = -(-w.T // 64)
    summ = torch.zeros((2, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(2, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=16, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(2)]).contiguous()
    out = dash.decode(q, k, v, lens_t, summ, sigma=2.0, enable_gqa=True)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    for b in range(2):
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        sigma=2.0, rows=[lens[b] - 1])
        compare_out(g[b], ref["out"][0, :, 0], "bf16", what=f"decode sigma b={b}")


@pytest.mark.parametrize("dtype,G,alpha", [("bf16", 16, 1.5), ("bf16", 4, 2.0), ("fp32", 8, 1.5)])
def test_decode_estimate_diagonal(dash, dtype, G, alpha):
    """dash_decode_diag with estimate_diagonal: each decode row equals the oracle's prefill
    row with the flag (mask bits outside the margin, outputs); lengths mid-chunk, at a chunk
    boundary, one past it, and in the first chunk."""
    T = 1500
    w = Workload(name=f"dec_diag_{dtype}", kind="prefill", B=4, Hq=2 * G, Hkv=2, T=T, D=128,
                 dtype=dtype, seed=960 + G, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    lens = [1500, 1024, 1025, 40]
    say(f"[parity] decode estimate_diagonal {dtype} G={G} alpha={alpha} lens={lens}")
    k, v, hc = (to_dev(x[n], dtype) for n in ("k", "v", "head_cls"))
    nc = -(-T // 64)
    summ = torch.zeros((4, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(4, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=2 * G, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], dtype) for b in range(4)]).contiguous()
    out, ab = dash.decode(q, k, v, lens_t, summ, alpha=alpha, enable_gqa=True,
                          estimate_diagonal=True, head_cls=hc, return_active_blocks=True)
    plain = dash.decode(q, k, v, lens_t, summ, alpha=alpha, enable_gqa=True)
    torch.cuda.synchronize()
    g, bits = out.float().cpu().numpy(), unpack_words(ab.cpu().numpy(), nc)
    moved = 0.0
    for b in range(4):
        t = lens[b] - 1
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        alpha=alpha, rows=[t], estimate_diagonal=True)
        compare_out(g[b], ref["out"][0, :, 0], dtype, what=f"decode diag b={b}")
        compare_mask(bits[b][None, :, None, :], ref["mask"], ref["margin"], [t])
        moved = max(moved, float((out[b].float() - plain[b].float()).abs().max()))
    assert moved > 1e-5        # the flag reaches the kernels (same inputs, deterministic)


@pytest.mark.parametrize("G,k,T,rows", [
    (16, 8, 2000, list(range(0, 2000, 7)) + [1999]),   # the 128K workload's head ratio
    (4, 1, 1100, None),                                 # argmax routing, every row
    (8, 40, 1500, list(range(0, 1500, 5)) + [1499]),   # k above the early rows' lengths
    (16, 64, 16384, [64, 4095, 9000, 16383]),
])
def test_prefill_topk_router(dash, G, k, T, rows):
    """The top-k comparison router: mask bits equal the oracle's outside the 1e-4 score
    margin, weight 1 at every set bit, and every row's output equals the oracle's attention
    over the chunks the GPU selected (equal to the oracle's own selection where no chunk
    sits within the margin of the k-th score)."""
    w = Workload(name=f"topk_g{G}", kind="prefill", B=1, Hq=2 * G, Hkv=2, T=T, D=128,
                 dtype="bf16", seed=970 + G, needle_amp=1.0)
    r = run_prefill(dash, w, rows=rows, topk=k)
    ref, rows = r["ref"], r["rows"]
    amb = compare_mask(r["bits"], ref["mask"], ref["margin"], rows)
    nc = r["nc"]
    # weights: exactly 1 at set bits, 0 elsewhere
    np.testing.assert_array_equal(r["w"][r["bits"][..., :r["w"].shape[-1]]], 1.0)
    # selection size: k per row (all routed chunks when there are at most k), ties aside
    for i, t in enumerate(rows):
        n = r["bits"][0, :, i, :t // 64].sum(axis=-1)
        assert np.all(n >= min(k, t // 64)), (t, n)
    # outputs against the oracle's attention over the GPU's own selection
    x = r["x"]
    scale = 1.0 / np.sqrt(w.D)
    err = 0.0
    for i, t in enumerate(rows):
        for kvh in range(w.Hkv):
            wb = r["bits"][0, kvh, i, :t // 64].astype(np.float64)
            for g in range(G):
                h = kvh * G + g
                o = O.attend_row(x["q"][0, h, t], x["k"][0, kvh], x["v"][0, kvh], int(t), wb,
                                 scale=scale)
                err = max(err, compare_out(r["out"][0, h, i], o, "bf16", what=f"topk row {t}"))
    flips = int((r["bits"][..., :nc] != ref["mask"]).sum())
    say(f"[parity]   topk k={k}: out err {err:.2e}, near-threshold flips {amb} (all flips {flips})")


@pytest.mark.parametrize("k", [1, 16, 200])
def test_decode_topk_router(dash, k):
    """Decode with the top-k comparison router: mask bits equal the oracle's prefill row
    outside the 1e-4 score margin, and the output equals the oracle's attention over the
    chunks the GPU selected."""
    w = Workload(name="dec_topk", kind="prefill", B=3, Hq=32, Hkv=2, T=9000, D=128,
                 dtype="bf16", seed=980, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say(f"[parity] decode top-{k}")
    kk, vv, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    lens = [9000, 4100, 700]
    nc = -(-w.T // 64)
    summ = torch.zeros((3, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(3, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(kk, hc, lens_t, summ, nsum, Hq=32, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(3)]).contiguous()
    out, ab = dash.decode(q, kk, vv, lens_t, summ, topk=k, enable_gqa=True,
                          return_active_blocks=True)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    bits = unpack_words(ab.cpu().numpy(), nc)
    scale = 1.0 / np.sqrt(128)
    for b in range(3):
        t = lens[b] - 1
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        rows=[t], topk=k)
        compare_mask(bits[b][:, None], ref["mask"][0], ref["margin"][0], [t])
        for kvh in range(2):
            wb = bits[b, kvh, :t // 64].astype(np.float64)
            assert wb.sum() >= min(k, t // 64)
            for hh in range(16):
                h = kvh * 16 + hh
                o = O.attend_row(x["q"][b, h, t], x["k"][b, kvh], x["v"][b, kvh], t, wb,
                                 scale=scale)
                compare_out(g[b, h], o, "bf16", what=f"decode topk b={b} h={h}")


def test_prefill_fp32_gqa_and_scale(dash):
    w = Workload(name="fp32_gqa", kind="prefill", B=1, Hq=8, Hkv=2, T=390, D=128,
                 dtype="fp32", gamma=2.0, seed=77, needle_amp=1.5)
    check_prefill(run_prefill(dash, w), w)


def test_prefill_16k_gqa_sampled_rows(dash):
    """The 16K, 32/8-head workload at full size, checked on sampled rows."""
    from long_context_sparse_stage0_amd.workloads import PREFILL_16K_GQA as w
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 63, 64, 65, 127, 128, w.T - 1],
                                     rng.integers(0, w.T, size=25)]))
    check_prefill(run_prefill(dash, w, rows=rows), w)


@pytest.mark.parametrize("dist", ["uniform", "left_outliers", "exp_left"])
def test_prefill_router_shaped_scores(dash, dist):
    """Chunk logits with a uniform, a left-outlier and a left-skewed distribution over
    300 chunks (16 heads): on rows past 256 routed chunks the router's Gaussian start point
    lies past the threshold for these shapes, so the fallback step decides the result."""
    T, D, G = 64 * 300, 128, 16
    x = synth.chunk_valued_prefill(T, D, G, dist, amp=2.0 * math.sqrt(D), seed=4242)
    say(f"[parity] prefill shaped scores {dist} T={T} G={G}")
    q, k, v, hc = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "head_cls"))
    out, ab, bw = dash.prefill(q, k, v, hc, alpha=1.5, enable_gqa=True,
                               return_active_blocks=True, return_block_weights=True)
    torch.cuda.synchronize()
    rows = np.array([64 * 200 + 5, 64 * 256, 64 * 256 + 63, 64 * 280 + 17, T - 1])
    ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=1.5, rows=rows)
    nc = -(-T // 64)
    e_out = compare_out(out.float().cpu().numpy()[:, :, rows], ref["out"], "bf16")
    e_w = compare_weights(bw.cpu().numpy()[:, :, rows], ref["w_bar"])
    amb = compare_mask(unpack_words(ab.cpu().numpy(), nc)[:, :, rows], ref["mask"],
                       ref["margin"], rows)
    frac = O.zero_fraction(ref["w_bar"], rows)
    say(f"[parity]   out err {e_out:.2e}  w err {e_w:.2e}  near-threshold flips {amb}  "
        f"zero-weight fraction {frac:.3f}")


def test_dense_causal_matches_textbook(dash):
    rng = np.random.default_rng(3)
    B, Hq, Hkv, T, D = 1, 4, 2, 300, 128
    q = synth.round_bf16(rng.normal(size=(B, Hq, T, D)))
    k = synth.round_bf16(rng.normal(size=(B, Hkv, T, D)))
    v = synth.round_bf16(rng.normal(size=(B, Hkv, T, D)))
    say("[parity] dense causal comparator T=300")
    out = dash.dense_causal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                            enable_gqa=True)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    for h in range(Hq):
        ref = O.causal_attention(q[0, h], k[0, h // 2], v[0, h // 2])
        compare_out(g[0, h], ref, "bf16", what=f"dense head {h}")


def _decode_case(dash, w, lens, check_rows=True):
    """Fill a cache with the first lens[b] tokens, build the summary cache with
    append_chunk, run one decode step, compare with the oracle's prefill row."""
    x = synth.prefill_inputs(w)
    B, Hkv, T, D = w.B, w.Hkv, w.T, w.D
    dev_k, dev_v = to_dev(x["k"], w.dtype), to_dev(x["v"], w.dtype)
    hc = to_dev(x["head_cls"], w.dtype)
    nc = -(-T // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(dev_k, hc, lens_t, summ, nsum, Hq=w.Hq, enable_gqa=w.enable_gqa)
    rows = [l - 1 for l in lens]
    qd = torch.stack([to_dev(x["q"][b, :, rows[b]], w.dtype) for b in range(B)])
    out, ab = dash.decode(qd.contiguous(), dev_k, dev_v, lens_t, summ, alpha=w.alpha,
                          enable_gqa=w.enable_gqa, return_active_blocks=True)
    torch.cuda.synchronize()
    assert nsum.cpu().tolist() == [l // 64 for l in lens]
    g = out.float().cpu().numpy()
    bits = unpack_words(ab.cpu().numpy(), nc)
    for b in range(B):
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        alpha=w.alpha, rows=[rows[b]])
        compare_out(g[b], ref["out"][0, :, 0], w.dtype, what=f"decode b={b}")
        compare_mask(bits[b][:, None], ref["mask"][0], ref["margin"][0], [rows[b]])


def test_decode_matches_prefill_rows(dash):
    w = Workload(name="dec_small", kind="prefill", B=3, Hq=32, Hkv=2, T=1300, D=128,
                 dtype="bf16", seed=31, needle_amp=1.0)
    say("[parity] decode vs prefill rows")
    _decode_case(dash, w, [1300, 640, 65])


def test_decode_fp32_and_invalid_len(dash):
    w = Workload(name="dec_fp32", kind="prefill", B=2, Hq=2, Hkv=2, T=700, D=64,
                 dtype="fp32", seed=32, q_mode="iid", needle_count="none")
    say("[parity] decode fp32")
    _decode_case(dash, w, [700, 129])
    # an out-of-range length gives NaN for that sequence only
    x = synth.prefill_inputs(w)
    k, v = to_dev(x["k"], "fp32"), to_dev(x["v"], "fp32")
    summ = torch.zeros((2, 2, 11, 64), dtype=torch.float32, device="cuda")
    lens = torch.tensor([701, 5], dtype=torch.int32, device="cuda")
    q = to_dev(x["q"][:, :, 4], "fp32").contiguous()
    out = dash.decode(q, k, v, lens, summ)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isnan(o[0]).all() and np.isfinite(o[1]).all()


def test_decode_bf16_segments_and_invalid_len(dash):
    """bf16 decode whose work lists split into several attend segments per (b, kv head),
    merged by log-sum-exp; two calls share one workspace that starts as garbage (nothing
    may carry over from the previous call); an out-of-range length gives NaN for that
    sequence only."""
    w = Workload(name="dec_segs", kind="prefill", B=2, Hq=16, Hkv=2, T=6000, D=128,
                 dtype="bf16", seed=35, needle_amp=0.5)
    x = synth.prefill_inputs(w)
    say("[parity] decode bf16 segments, shared workspace, invalid length")
    B, Hkv, T, D = w.B, w.Hkv, w.T, w.D
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    nc = -(-T // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, torch.full((B,), T, dtype=torch.int32, device="cuda"), summ, nsum,
                      Hq=w.Hq, enable_gqa=True)
    p = dash.make_params(B, w.Hq, Hkv, T, D, alpha=w.alpha, enable_gqa=True,
                         dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("decode", p), "cuda")
    ws.fill_(0xA5)                                   # garbage before the first call
    for lens in ([T, 4097], [5000, T + 1]):
        rows = [min(l, T) - 1 for l in lens]
        q = torch.stack([to_dev(x["q"][b, :, rows[b]], "bf16") for b in range(B)]).contiguous()
        lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
        out, ab = dash.decode(q, k, v, lens_t, summ, alpha=w.alpha, enable_gqa=True,
                              workspace=ws, return_active_blocks=True)
        torch.cuda.synchronize()
        g = out.float().cpu().numpy()
        bits = unpack_words(ab.cpu().numpy(), nc)
        for b in range(B):
            if lens[b] > T:
                assert np.isnan(g[b]).all(), f"b={b}: out-of-range length must give NaN"
                continue
            ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                            alpha=w.alpha, rows=[rows[b]])
            active = int(ref["mask"][0][:, 0].sum(axis=-1).min())   # per kv head
            assert active + 1 > 16, f"b={b}: {active} active chunks give one segment only"
            compare_out(g[b], ref["out"][0, :, 0], "bf16", what=f"decode segs b={b}")
            compare_mask(bits[b][:, None], ref["mask"][0], ref["margin"][0], [rows[b]])


def _page_pool(cache, perm, num_pages, lens, gen):
    """Scatter a contiguous cache [B, Hkv, T, D] into a page pool [num_pages, Hkv, 64, D]:
    chunk c of sequence b goes to page perm[b * nc + c]; spare pages hold noise."""
    B, Hkv, T, D = cache.shape
    nc = -(-T // 64)
    padded = torch.zeros((B, Hkv, nc * 64, D), dtype=cache.dtype, device=cache.device)
    padded[:, :, :T] = cache
    chunks = padded.view(B, Hkv, nc, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nc, Hkv, 64, D)
    pool = torch.randn((num_pages, Hkv, 64, D), generator=gen, device="cpu").to(cache.dtype)
    pool = pool.to(cache.device)
    pool[torch.as_tensor(perm, device=cache.device)] = chunks
    table = torch.as_tensor(np.asarray(perm, np.int32).reshape(B, nc)).clone()
    for b, L in enumerate(lens):                       # entries past a length are never read
        table[b, -(-L // 64):] = -1
    return pool, table.to(cache.device)


def test_decode_paged_matches_contiguous(dash):
    """Paged caches (shuffled pages, noise in the spare ones): the summary append and the
    decode step give bit-identical results to the contiguous caches, and equal the
    oracle's prefill rows."""
    w = Workload(name="dec_paged", kind="prefill", B=3, Hq=16, Hkv=2, T=1500, D=128,
                 dtype="bf16", seed=960, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say("[parity] paged decode vs contiguous")
    B, Hkv, T, D = w.B, w.Hkv, w.T, w.D
    lens = [1500, 900, 130]
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    nc = -(-T // 64)
    rng = np.random.default_rng(961)
    num_pages = B * nc + 7
    perm = rng.permutation(num_pages)[:B * nc]
    gen = torch.Generator().manual_seed(962)
    kp, table = _page_pool(k, perm, num_pages, lens, gen)
    vp, _ = _page_pool(v, perm, num_pages, lens, gen)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    s_c = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    s_p = torch.zeros_like(s_c)
    n_c = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_p = torch.zeros_like(n_c)
    dash.append_chunk(k, hc, lens_t, s_c, n_c, Hq=w.Hq, enable_gqa=True)
    dash.append_chunk_paged(kp, table, hc, lens_t, s_p, n_p, Hq=w.Hq, enable_gqa=True)
    torch.cuda.synchronize()
    assert torch.equal(s_c, s_p) and torch.equal(n_c, n_p)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(B)]).contiguous()
    o_c, ab_c = dash.decode(q, k, v, lens_t, s_c, enable_gqa=True, return_active_blocks=True)
    o_p, ab_p = dash.decode_paged(q, kp, vp, table, lens_t, s_p, enable_gqa=True,
                                  return_active_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_p)
    W = ab_c.shape[-1]
    assert torch.equal(ab_c, ab_p[..., :W])
    g = o_p.float().cpu().numpy()
    for b in range(B):
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        rows=[lens[b] - 1])
        compare_out(g[b], ref["out"][0, :, 0], "bf16", what=f"paged decode b={b}")


def test_decode_many_sequences(dash):
    """More (b, kv head) pairs than attend workgroup slots (300 sequences of mixed lengths,
    2 KV heads): every list is one segment; sampled sequences equal the oracle's rows."""
    B, T = 300, 400
    w = Workload(name="dec_many", kind="prefill", B=B, Hq=8, Hkv=2, T=T, D=128, dtype="bf16",
                 seed=36, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say(f"[parity] decode with {B} sequences")
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    rng = np.random.default_rng(37)
    lens = rng.integers(1, T + 1, size=B)
    lens[:4] = [T, 1, 64, 129]
    nc = -(-T // 64)
    summ = torch.zeros((B, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=8, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(B)]).contiguous()
    out, ab = dash.decode(q, k, v, lens_t, summ, enable_gqa=True, return_active_blocks=True)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    bits = unpack_words(ab.cpu().numpy(), nc)
    for b in list(range(4)) + list(rng.choice(np.arange(4, B), size=12, replace=False)):
        t = int(lens[b]) - 1
        ref = O.prefill(x["q"][b:b + 1], x["k"][b:b + 1], x["v"][b:b + 1], x["head_cls"],
                        rows=[t])
        compare_out(g[b], ref["out"][0, :, 0], "bf16", what=f"decode b={b} len={t + 1}")
        compare_mask(bits[b][:, None], ref["mask"][0], ref["margin"][0], [t])


def test_decode_paged_with_options(dash):
    """The options compose: paged caches with the top-k router, with a prior strength
    sigma != 1 and with estimate_diagonal give outputs and masks bit-identical to the
    contiguous caches."""
    w = Workload(name="dec_paged_opts", kind="prefill", B=2, Hq=16, Hkv=2, T=2200, D=128,
                 dtype="bf16", seed=965, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say("[parity] paged decode with top-k and sigma")
    B, Hkv, T, D = w.B, w.Hkv, w.T, w.D
    lens = [2200, 1400]
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    nc = -(-T // 64)
    rng = np.random.default_rng(966)
    num_pages = B * nc + 3
    perm = rng.permutation(num_pages)[:B * nc]
    gen = torch.Generator().manual_seed(967)
    kp, table = _page_pool(k, perm, num_pages, lens, gen)
    vp, _ = _page_pool(v, perm, num_pages, lens, gen)
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=w.Hq, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(B)]).contiguous()
    for opts in (dict(topk=12), dict(sigma=0.5), dict(topk=5, sigma=2.0),
                 dict(estimate_diagonal=True, head_cls=hc),
                 dict(estimate_diagonal=True, head_cls=hc, sigma=0.5)):
        o_c, a_c = dash.decode(q, k, v, lens_t, summ, enable_gqa=True, return_active_blocks=True,
                               **opts)
        o_p, a_p = dash.decode_paged(q, kp, vp, table, lens_t, summ, enable_gqa=True,
                                     return_active_blocks=True, **opts)
        torch.cuda.synchronize()
        assert torch.equal(o_c, o_p), list(opts)
        assert torch.equal(a_c, a_p[..., :a_c.shape[-1]]), list(opts)


def test_decode_steps_with_append(dash):
    """Decode 100 consecutive steps from a 600-token prompt (GQA 4), appending each chunk
    as it fills; every step equals the oracle's prefill row of the full sequence."""
    w = Workload(name="dec_steps", kind="prefill", B=2, Hq=8, Hkv=2, T=700, D=128,
                 dtype="bf16", seed=33, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say("[parity] decode 100 steps with appends, GQA 4")
    k, v, hc = to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"), to_dev(x["head_cls"], "bf16")
    B, Hkv, T, D = 2, 2, 700, 128
    nc = -(-T // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    L0 = 600
    dash.append_chunk(k, hc, torch.full((B,), L0, dtype=torch.int32, device="cuda"), summ, nsum,
                      Hq=8, enable_gqa=True)
    outs = []
    for s in range(T - L0):
        L = L0 + s + 1
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        q = to_dev(x["q"][:, :, L - 1], "bf16").contiguous()
        outs.append(dash.decode(q, k, v, lens, summ, enable_gqa=True).float().cpu().numpy())
        if L % 64 == 0:
            dash.append_chunk(k, hc, lens, summ, nsum, Hq=8, enable_gqa=True)
    torch.cuda.synchronize()
    rows = np.arange(L0, T)
    ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], rows=rows)
    g = np.stack(outs, axis=2)                       # [B, Hq, steps, D]
    compare_out(g, ref["out"], "bf16", what="decode steps")


@pytest.mark.parametrize("T,dtype,G", [(1, "bf16", 4), (63, "bf16", 16), (64, "bf16", 2),
                                       (65, "bf16", 8), (1, "fp32", 1), (64, "fp32", 2),
                                       (129, "fp32", 4)])
def test_prefill_tiny_sequences(dash, T, dtype, G):
    """Degenerate lengths: a single token, rows that have no routed chunk at all, and the
    first row that routes over exactly one chunk."""
    w = Workload(name=f"tiny_{T}", kind="prefill", B=2, Hq=2 * G, Hkv=2, T=T, D=64,
                 dtype=dtype, seed=700 + T, needle_amp=1.0)
    check_prefill(run_prefill(dash, w), w)


def test_decode_short_sequences(dash):
    """Decode rows with one token in the cache, a full first chunk (no routed chunk yet) and
    the first row that routes over one chunk."""
    w = Workload(name="dec_short", kind="prefill", B=3, Hq=8, Hkv=2, T=200, D=128,
                 dtype="bf16", seed=34, needle_amp=1.0)
    say("[parity] decode short sequences")
    _decode_case(dash, w, [1, 64, 65])
