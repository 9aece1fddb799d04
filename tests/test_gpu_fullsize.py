"""GPU parity at full size: the 128K prefill workload in the launch configuration the
benchmark times, the longest supported sequence (2049 chunks, 2048 routed chunks on the
last row), and the 64K decode workload over all 256 steps with summary appends.  The
oracle checks sampled rows / steps; inputs are the seeded generator's, expected values
come only from the oracle."""
import numpy as np
import pytest

from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import (DECODE_64K_B16, PREFILL_128K_GQA,
                                                      Workload)
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


def _sample_rows(T, n, seed, fixed):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.asarray(fixed), rng.integers(0, T, size=n)])
    return np.unique(rows[(rows >= 0) & (rows < T)])


def _prefill_bench_config(dash, w, rows, estimate_diagonal=False):
    """Run the prefill exactly as the benchmark does (Stages 0, 1, 2 on one workspace),
    then again with the block weights returned; compare sampled rows with the oracle."""
    x = synth.prefill_inputs(w)
    say(f"[fullsize] prefill {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
        f"rows={len(rows)}")
    q, k, v, hc = (to_dev(x[n], w.dtype) for n in ("q", "k", "v", "head_cls"))
    B, Hkv, T = w.B, w.Hkv, w.T
    nc = -(-T // 64)
    W = -(-nc // 64)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    p = dash.make_params(B, w.Hq, Hkv, T, w.D, alpha=w.alpha, gamma=w.gamma,
                         enable_gqa=w.enable_gqa, dtype=dt)
    ws = dash.alloc_workspace(dash.workspace_size("prefill", p), "cuda")
    out = torch.empty_like(q)
    ab = torch.empty((B, Hkv, T, W), dtype=torch.int64, device="cuda")
    kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=w.enable_gqa,
              estimate_diagonal=estimate_diagonal)
    for s in (0, 3, 1, 2):                   # the timed step of the benchmark
        dash.prefill_stage(s, q, k, v, hc, out, ws, **kw)
    # the mask as the benchmark reads it (Stage 1 again, mask into the caller's buffer)
    dash.prefill_stage(1, q, k, v, hc, out, ws, active_blocks=ab, **kw)
    torch.cuda.synchronize()
    ridx = torch.as_tensor(rows, device="cuda")
    g_out = out.index_select(2, ridx).float().cpu().numpy()
    g_bits = unpack_words(ab.index_select(2, ridx).cpu().numpy(), nc)
    del ab
    # same kernels with the weights returned: the output must be bit-identical
    out2, bw = dash.prefill(q, k, v, hc, return_block_weights=True, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2.index_select(2, ridx), out.index_select(2, ridx))
    g_w = bw.index_select(2, ridx).cpu().numpy()
    del bw, out, out2, q, k, v, ws
    torch.cuda.empty_cache()
    summ = O.chunk_summaries(x["k"], x["head_cls"], 1.0 / np.sqrt(w.D))
    ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=w.alpha, gamma=w.gamma,
                    rows=rows, summaries=summ, estimate_diagonal=estimate_diagonal)
    e_out = compare_out(g_out, ref["out"], w.dtype)
    e_w = compare_weights(g_w, ref["w_bar"])
    amb = compare_mask(g_bits, ref["mask"], ref["margin"], rows)
    frac = O.zero_fraction(ref["w_bar"], rows)
    say(f"[fullsize]   out err {e_out:.2e}  w err {e_w:.2e}  near-threshold flips {amb}  "
        f"zero-weight fraction (sampled rows) {frac:.3f}")
    return frac


def test_prefill_128k_sampled_rows(dash):
    """The 128K workload (32/2 heads, calibrated needles) on 30 sampled rows, including the
    first and last rows of chunks and the final row (2047 routed chunks)."""
    w = PREFILL_128K_GQA
    rows = _sample_rows(w.T, 20, 1, [0, 63, 64, 65, 4095, 65536, 131007, 131008, w.T - 1])
    frac = _prefill_bench_config(dash, w, rows)
    assert 0.5 < frac < 0.95


def test_prefill_128k_estimate_diagonal(dash):
    """The 128K workload with estimate_diagonal (the own chunk's partial summary in every
    head's entmax, on the MFMA router) on sampled rows: first, middle and last rows of chunks
    and the final row."""
    w = PREFILL_128K_GQA
    rows = _sample_rows(w.T, 8, 3, [64, 65, 127, 65536 + 31, 131008, w.T - 1])
    _prefill_bench_config(dash, w, rows, estimate_diagonal=True)


def test_prefill_longest_sequence(dash):
    """T = 64 * 2049: the last row routes over the maximum of 2048 chunks (bf16, G = 2)."""
    w = Workload(name="longest", kind="prefill", B=1, Hq=4, Hkv=2, T=64 * 2049, D=128,
                 dtype="bf16", seed=41, needle_amp=1.0)
    rows = _sample_rows(w.T, 6, 2, [64 * 2048 - 1, 64 * 2048, w.T - 2, w.T - 1])
    _prefill_bench_config(dash, w, rows)


def test_decode_longest_sequence(dash):
    """Decode at the longest supported sequence (2049 chunks, the last row routing over 2048):
    the largest solver register set, and (with one sequence) more attend segments than the
    combine kernel's first round of loads holds; equals the oracle's prefill row."""
    T = 64 * 2049
    w = Workload(name="dec_longest", kind="prefill", B=1, Hq=32, Hkv=2, T=T, D=128,
                 dtype="bf16", seed=990, needle_amp=0.5)
    x = synth.prefill_inputs(w)
    say(f"[fullsize] decode at T = {T}")
    k, v, hc = (to_dev(x[n], "bf16") for n in ("k", "v", "head_cls"))
    nc = -(-T // 64)
    summ = torch.zeros((1, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(1, dtype=torch.int32, device="cuda")
    for L in (T, T - 100):
        lens = torch.tensor([L], dtype=torch.int32, device="cuda")
        summ.zero_()
        nsum.zero_()
        dash.append_chunk(k, hc, lens, summ, nsum, Hq=32, enable_gqa=True)
        q = to_dev(x["q"][:, :, L - 1], "bf16").contiguous()
        out, ab = dash.decode(q, k, v, lens, summ, enable_gqa=True, return_active_blocks=True)
        torch.cuda.synchronize()
        ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], rows=[L - 1])
        e = compare_out(out.float().cpu().numpy()[0], ref["out"][0, :, 0], "bf16",
                        what=f"decode at {L}")
        bits = unpack_words(ab.cpu().numpy(), nc)
        amb = compare_mask(bits[0][:, None], ref["mask"][0], ref["margin"][0], [L - 1])
        act = bits[0].sum(axis=-1)                            # per kv head
        say(f"[fullsize]   L={L}: out err {e:.2e}, near-threshold flips {amb}, "
            f"active chunks {act.tolist()}")
        if L == T:     # a list longer than 16 segments of 16 items
            assert int(act.max()) + 1 > 16 * 16, act


def test_decode_64k_all_steps_sampled(dash):
    """The 64K decode workload (B = 16, 32/2 heads): all 256 steps in order, appending a
    summary whenever a chunk fills; steps around the append are checked in full against the
    oracle's decode step, which uses its own summaries of the same cache."""
    w = DECODE_64K_B16
    x = synth.decode_inputs(w)
    say(f"[fullsize] decode {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} cache={w.T} steps={w.steps}")
    kc, vc, hc = (to_dev(x[n], "bf16") for n in ("k_cache", "v_cache", "head_cls"))
    qs = to_dev(x["q_steps"], "bf16")
    B, Hkv, TT, D = kc.shape
    Hq = qs.shape[2]
    nc = -(-TT // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    dash.append_chunk(kc, hc, torch.full((B,), w.T, dtype=torch.int32, device="cuda"), summ,
                      nsum, Hq=Hq, enable_gqa=True)
    p = dash.make_params(B, Hq, Hkv, TT, D, alpha=w.alpha, enable_gqa=True,
                         dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("decode", p), "cuda")
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    check = {0: None, 62: None, 63: None, 64: None, w.steps - 1: None}
    for s in range(w.steps):
        L = w.T + 1 + s
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o, ab = dash.decode(qs[s], kc, vc, lens, summ, alpha=w.alpha, enable_gqa=True, out=out,
                            workspace=ws, return_active_blocks=True)
        if s in check:
            check[s] = (o.float().cpu().numpy(), ab.cpu().numpy())
        if L % 64 == 0:
            dash.append_chunk(kc, hc, lens, summ, nsum, Hq=Hq, enable_gqa=True)
    torch.cuda.synchronize()
    assert nsum.cpu().tolist() == [(w.T + w.steps) // 64] * B
    del kc, vc, qs, summ, ws
    torch.cuda.empty_cache()
    o_summ = O.chunk_summaries(x["k_cache"], x["head_cls"], 1.0 / np.sqrt(D))
    for s, (g_o, g_ab) in check.items():
        L = w.T + 1 + s
        ref = O.decode_step(x["q_steps"][s], x["k_cache"], x["v_cache"], np.full(B, L), o_summ,
                            alpha=w.alpha)
        e = compare_out(g_o, ref["out"], "bf16", what=f"decode step {s}")
        bits = unpack_words(g_ab, nc)                       # [B, Hkv, nc]
        amb = compare_mask(bits[:, :, None, :], ref["mask"][:, :, None, :],
                           ref["margin"][:, :, None, :], [L - 1])
        act = float(bits.sum()) / (B * Hkv * ((L - 1) // 64))
        say(f"[fullsize]   step {s}: out err {e:.2e}, near-threshold flips {amb}, "
            f"active fraction {act:.3f}")


def test_decode_64k_paged_equals_contiguous(dash):
    """The 64K decode workload over paged caches (every chunk of every sequence in a
    shuffled page of one pool): 24 steps across a chunk boundary with the paged append give
    outputs and masks bit-identical to the contiguous caches."""
    w = DECODE_64K_B16
    x = synth.decode_inputs(w)
    say(f"[fullsize] paged decode {w.name} B={w.B}")
    kc, vc, hc = (to_dev(x[n], "bf16") for n in ("k_cache", "v_cache", "head_cls"))
    qs = to_dev(x["q_steps"][40:64 + 40], "bf16")        # steps 40..63 cross a chunk boundary
    del x
    B, Hkv, TT, D = kc.shape
    Hq = qs.shape[2]
    nc = -(-TT // 64)
    perm = torch.randperm(B * nc, generator=torch.Generator().manual_seed(77)).cuda()

    def pages(cache):
        pad = torch.zeros((B, Hkv, nc * 64, D), dtype=cache.dtype, device="cuda")
        pad[:, :, :TT] = cache
        pool = torch.empty((B * nc, Hkv, 64, D), dtype=cache.dtype, device="cuda")
        pool[perm] = pad.view(B, Hkv, nc, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nc, Hkv, 64, D)
        return pool
    kp, vp = pages(kc), pages(vc)
    table = perm.view(B, nc).to(torch.int32).contiguous()
    L0 = w.T + 40
    s_c = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    s_p = torch.zeros_like(s_c)
    n_c = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_p = torch.zeros_like(n_c)
    init = torch.full((B,), L0, dtype=torch.int32, device="cuda")
    dash.append_chunk(kc, hc, init, s_c, n_c, Hq=Hq, enable_gqa=True)
    dash.append_chunk_paged(kp, table, hc, init, s_p, n_p, Hq=Hq, enable_gqa=True)
    for s in range(24):
        L = L0 + 1 + s
        lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
        o_c, a_c = dash.decode(qs[s], kc, vc, lens, s_c, alpha=w.alpha, enable_gqa=True,
                               return_active_blocks=True)
        o_p, a_p = dash.decode_paged(qs[s], kp, vp, table, lens, s_p, alpha=w.alpha,
                                     enable_gqa=True, return_active_blocks=True)
        assert torch.equal(o_c, o_p), f"step {s}: outputs differ"
        assert torch.equal(a_c, a_p[..., :a_c.shape[-1]]), f"step {s}: masks differ"
        if L % 64 == 0:
            dash.append_chunk(kc, hc, lens, s_c, n_c, Hq=Hq, enable_gqa=True)
            dash.append_chunk_paged(kp, table, hc, lens, s_p, n_p, Hq=Hq, enable_gqa=True)
    torch.cuda.synchronize()
    assert torch.equal(s_c, s_p) and torch.equal(n_c, n_p)


@pytest.mark.parametrize("alpha,lam", [(1.25, 32.0), (2.0, 2.0)])
def test_sweep_64k_sampled_rows(dash, alpha, lam):
    """Two corners of the 64K sparsity sweep (32/8 heads, Poisson needle counts): the
    densest (alpha = 1.25, 32 needles per block) and the sparsest (alpha = 2, 2 needles)."""
    from long_context_sparse_stage0_amd.workloads import sweep_cell
    w = sweep_cell(alpha, lam)
    rows = _sample_rows(w.T, 10, 3, [64, 32768, w.T - 1])
    _prefill_bench_config(dash, w, rows)
