"""GPU parity on the configurations as they are timed: the dense comparator in the launch
instance the benchmark uses (32 query / 2 KV heads), the 16K workload on every row, the
128K workload on whole 64-row blocks (Stage 2 computes a block's rows together over the
union of their masks), every cell of the 64K sparsity sweep, decode with
estimate_diagonal on long rows, and a decode state saved to the host and restored
mid-run.  Expected values come only from the oracle, on the seeded generator's inputs."""
import numpy as np
import pytest

from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import (PREFILL_16K_GQA, PREFILL_128K_GQA,
                                                      Workload, sweep_cell)
from oracle import dash_oracle as O
from tests.parity_util import (compare_mask, compare_out, compare_weights, oracle_all_rows,
                               say, to_dev, unpack_words)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_stage0_amd import dash as d
    d.load()
    return d


# ---------------------------------------------------------------- dense comparator

@pytest.mark.parametrize("T,D", [(1000, 128), (1000, 64), (64, 128), (130, 64)])
def test_dense_causal_gqa16_every_row(dash, T, D):
    """The dense comparator at 32 query / 2 KV heads (the 8-wave launch instance the
    benchmark times) on every row of a ragged sequence, against textbook causal
    attention."""
    rng = np.random.default_rng(100 + T + D)
    B, Hq, Hkv = 1, 32, 2
    q = synth.round_bf16(rng.normal(size=(B, Hq, T, D)))
    k = synth.round_bf16(rng.normal(size=(B, Hkv, T, D)))
    v = synth.round_bf16(rng.normal(size=(B, Hkv, T, D)))
    say(f"[configs] dense causal G=16 T={T} D={D}")
    out = dash.dense_causal(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                            enable_gqa=True)
    torch.cuda.synchronize()
    g = out.float().cpu().numpy()
    err = 0.0
    for h in range(Hq):
        ref = O.causal_attention(q[0, h], k[0, h // 16], v[0, h // 16])
        err = max(err, compare_out(g[0, h], ref, "bf16", what=f"dense head {h}"))
    say(f"[configs]   max-abs error {err:.2e}")


def test_dense_causal_16k_sampled_rows(dash):
    """The dense comparator on the 16K shape at 32/2 heads: sampled rows (first and last
    rows of chunks, the final row) against the oracle's attention with every chunk active
    and a uniform prior, which equals textbook causal attention."""
    w = Workload(name="dense16k", kind="prefill", B=1, Hq=32, Hkv=2, T=16384, D=128,
                 dtype="bf16", seed=101, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    say("[configs] dense causal 16K, 32/2 heads")
    out = dash.dense_causal(*(to_dev(x[n], "bf16") for n in ("q", "k", "v")), enable_gqa=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 63, 64, 8191, 8192, w.T - 1],
                                     rng.integers(0, w.T, size=10)]))
    g = out.float().cpu().numpy()[:, :, rows]
    del out
    err = 0.0
    scale = 1.0 / np.sqrt(w.D)
    for i, t in enumerate(rows):
        ones = np.ones(int(t) // 64)
        for h in range(w.Hq):
            o = O.attend_row(x["q"][0, h, t], x["k"][0, h // 16], x["v"][0, h // 16], int(t),
                             ones, scale=scale)
            err = max(err, compare_out(g[0, h, i], o, "bf16", what=f"dense row {t} head {h}"))
    say(f"[configs]   max-abs error {err:.2e} over {len(rows)} rows")


# ---------------------------------------------------------------- 16K, every row

def test_prefill_16k_every_row(dash):
    """The 16K workload (32/8 heads, needles at +3 sigma) on all 16384 rows: outputs,
    block weights and mask bits; the oracle's rows are spread over worker processes."""
    w = PREFILL_16K_GQA
    x = synth.prefill_inputs(w)
    say(f"[configs] prefill {w.name}, every row")
    q, k, v, hc = (to_dev(x[n], "bf16") for n in ("q", "k", "v", "head_cls"))
    out, ab, bw = dash.prefill(q, k, v, hc, alpha=w.alpha, enable_gqa=True,
                               return_active_blocks=True, return_block_weights=True)
    torch.cuda.synchronize()
    nc = -(-w.T // 64)
    g_out = out.float().cpu().numpy()
    g_bits = unpack_words(ab.cpu().numpy(), nc)
    g_w = bw.cpu().numpy()
    del q, k, v, hc, out, ab, bw, x
    torch.cuda.empty_cache()
    ref_out, ref_w, ref_m, ref_mask = oracle_all_rows(w)
    rows = np.arange(w.T)
    e_out = compare_out(g_out, ref_out, "bf16")
    e_w = compare_weights(g_w, ref_w)
    amb = compare_mask(g_bits, ref_mask, ref_m, rows)
    say(f"[configs]   out err {e_out:.2e}  w err {e_w:.2e}  near-threshold flips {amb}  "
        f"zero-weight fraction {O.zero_fraction(ref_w, rows):.3f}")


# ---------------------------------------------------------------- 128K and the sweep

def _bench_config_rows(dash, w, rows):
    """Prefill as the benchmark runs it (Stages 0, 1, 2 on one workspace), the mask read
    back by Stage 1, the weights by a full call; sampled rows against the oracle."""
    x = synth.prefill_inputs(w)
    say(f"[configs] prefill {w.name} rows={len(rows)}")
    q, k, v, hc = (to_dev(x[n], w.dtype) for n in ("q", "k", "v", "head_cls"))
    B, Hkv, T = w.B, w.Hkv, w.T
    nc = -(-T // 64)
    W = -(-nc // 64)
    p = dash.make_params(B, w.Hq, Hkv, T, w.D, alpha=w.alpha, gamma=w.gamma,
                         enable_gqa=w.enable_gqa, dtype=torch.bfloat16)
    ws = dash.alloc_workspace(dash.workspace_size("prefill", p), "cuda")
    out = torch.empty_like(q)
    ab = torch.empty((B, Hkv, T, W), dtype=torch.int64, device="cuda")
    kw = dict(alpha=w.alpha, gamma=w.gamma, enable_gqa=w.enable_gqa)
    for s in (0, 3, 1, 2):
        dash.prefill_stage(s, q, k, v, hc, out, ws, **kw)
    dash.prefill_stage(1, q, k, v, hc, out, ws, active_blocks=ab, **kw)
    torch.cuda.synchronize()
    ridx = torch.as_tensor(rows, device="cuda")
    g_out = out.index_select(2, ridx).float().cpu().numpy()
    g_bits = unpack_words(ab.index_select(2, ridx).cpu().numpy(), nc)
    del ab
    out2, bw = dash.prefill(q, k, v, hc, return_block_weights=True, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out2.index_select(2, ridx), out.index_select(2, ridx))
    g_w = bw.index_select(2, ridx).cpu().numpy()
    del bw, out, out2, q, k, v, ws
    torch.cuda.empty_cache()
    summ = O.chunk_summaries(x["k"], x["head_cls"], 1.0 / np.sqrt(w.D))
    ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], alpha=w.alpha, gamma=w.gamma,
                    rows=rows, summaries=summ)
    e_out = compare_out(g_out, ref["out"], w.dtype)
    e_w = compare_weights(g_w, ref["w_bar"])
    amb = compare_mask(g_bits, ref["mask"], ref["margin"], rows)
    frac = O.zero_fraction(ref["w_bar"], rows)
    say(f"[configs]   out err {e_out:.2e}  w err {e_w:.2e}  near-threshold flips {amb}  "
        f"zero-weight fraction {frac:.3f}")
    return frac


def test_prefill_128k_whole_blocks(dash):
    """The 128K workload on two whole 64-row blocks, the middle one and the last one
    (2047 routed chunks), in the benchmark's launch configuration."""
    rows = np.concatenate([np.arange(65536, 65536 + 64), np.arange(131008, 131072)])
    frac = _bench_config_rows(dash, PREFILL_128K_GQA, rows)
    assert 0.5 < frac < 0.95


@pytest.mark.parametrize("alpha,lam", [(1.25, 2.0), (1.25, 8.0), (1.5, 2.0), (1.5, 8.0),
                                       (1.5, 32.0), (2.0, 8.0), (2.0, 32.0)])
def test_sweep_64k_cell(dash, alpha, lam):
    """The remaining cells of the 64K sparsity sweep (32/8 heads, Poisson needle counts;
    the two corners are checked with the full-size tests): sampled rows including the
    first row past 256 routed chunks, where the alpha = 1.5 solver takes its moment-based
    start."""
    w = sweep_cell(alpha, lam)
    rng = np.random.default_rng(int(alpha * 100) + int(lam))
    rows = np.unique(np.concatenate([[64, 64 * 256, 64 * 256 + 63, 32768, w.T - 1],
                                     rng.integers(0, w.T, size=8)]))
    _bench_config_rows(dash, w, rows)


# ---------------------------------------------------------------- decode

def test_decode_estimate_diagonal_long_rows(dash):
    """Decode with estimate_diagonal on the 128K workload's sequence at lengths routing
    over 300, 1100 and 2047 chunks (the alpha = 1.5 moment-based start, the largest solver
    register sets): outputs and mask bits against the oracle's prefill rows with the flag;
    then the same step over paged caches is bit-identical."""
    w = PREFILL_128K_GQA
    x = synth.prefill_inputs(w)
    lens = [300 * 64 + 18, 1100 * 64 + 41, w.T]
    B = len(lens)
    say(f"[configs] decode estimate_diagonal lens={lens}")
    k1, v1, hc = (to_dev(x[n], "bf16") for n in ("k", "v", "head_cls"))
    k = k1.expand(B, -1, -1, -1).contiguous()
    v = v1.expand(B, -1, -1, -1).contiguous()
    del k1, v1
    Hkv, T, D = w.Hkv, w.T, w.D
    nc = -(-T // 64)
    summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=w.Hq, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][0, :, L - 1], "bf16") for L in lens]).contiguous()
    out, ab = dash.decode(q, k, v, lens_t, summ, enable_gqa=True, estimate_diagonal=True,
                          head_cls=hc, return_active_blocks=True)
    torch.cuda.synchronize()
    g, bits = out.float().cpu().numpy(), unpack_words(ab.cpu().numpy(), nc)
    # the same step over paged caches (chunks in shuffled pages)
    perm = torch.randperm(B * nc, generator=torch.Generator().manual_seed(11)).cuda()

    def pages(cache):
        pool = torch.empty((B * nc, Hkv, 64, D), dtype=cache.dtype, device="cuda")
        pool[perm] = cache.view(B, Hkv, nc, 64, D).permute(0, 2, 1, 3, 4).reshape(B * nc, Hkv, 64, D)
        return pool
    kp, vp = pages(k), pages(v)
    table = perm.view(B, nc).to(torch.int32).contiguous()
    o_p, a_p = dash.decode_paged(q, kp, vp, table, lens_t, summ, enable_gqa=True,
                                 estimate_diagonal=True, head_cls=hc, return_active_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o_p) and torch.equal(ab, a_p[..., :ab.shape[-1]])
    del k, v, kp, vp, summ
    torch.cuda.empty_cache()
    summ_o = O.chunk_summaries(x["k"], x["head_cls"], 1.0 / np.sqrt(D))
    for b, L in enumerate(lens):
        t = L - 1
        ref = O.prefill(x["q"], x["k"], x["v"], x["head_cls"], rows=[t], summaries=summ_o,
                        estimate_diagonal=True)
        e = compare_out(g[b], ref["out"][0, :, 0], "bf16", what=f"decode diag len {L}")
        amb = compare_mask(bits[b][None, :, None, :], ref["mask"], ref["margin"], [t])
        say(f"[configs]   len {L} (routed {t // 64}): out err {e:.2e}, near-threshold flips "
            f"{amb}, active {bits[b].sum(axis=-1).tolist()}")


def test_decode_state_save_restore(dash):
    """A decode run of 256 steps (4 sequences, 32/2 heads, chunk appends) stopped after 128
    steps, its state (K/V caches, summary cache, summarised-chunk counts) copied to the host,
    freed, restored into new device buffers and continued for 128 steps gives outputs and a
    final state bit-identical to the uninterrupted run.  Summaries are frozen once their
    chunk is complete, so nothing is recomputed on restore."""
    w = Workload(name="dec_resume", kind="decode", B=4, Hq=32, Hkv=2, T=4000, D=128,
                 dtype="bf16", seed=555, needle_amp=0.5, steps=256)
    x = synth.decode_inputs(w)
    say("[configs] decode save/restore, 128 + 128 steps")
    B, Hkv, TT, D = x["k_cache"].shape
    full_k, full_v = to_dev(x["k_cache"], "bf16"), to_dev(x["v_cache"], "bf16")
    hc = to_dev(x["head_cls"], "bf16")
    qs = to_dev(x["q_steps"], "bf16")
    nc = -(-TT // 64)

    def fresh_state():
        k = torch.zeros_like(full_k)
        v = torch.zeros_like(full_v)
        k[:, :, :w.T] = full_k[:, :, :w.T]
        v[:, :, :w.T] = full_v[:, :, :w.T]
        summ = torch.zeros((B, Hkv, nc, D), dtype=torch.float32, device="cuda")
        nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
        dash.append_chunk(k, hc, torch.full((B,), w.T, dtype=torch.int32, device="cuda"),
                          summ, nsum, Hq=w.Hq, enable_gqa=True)
        return {"k": k, "v": v, "summ": summ, "nsum": nsum}

    def run(st, s0, s1, outs):
        for s in range(s0, s1):
            L = w.T + 1 + s
            st["k"][:, :, L - 1] = full_k[:, :, L - 1]        # the new token's key and value
            st["v"][:, :, L - 1] = full_v[:, :, L - 1]
            lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
            outs.append(dash.decode(qs[s], st["k"], st["v"], lens, st["summ"], enable_gqa=True))
            if L % 64 == 0:
                dash.append_chunk(st["k"], hc, lens, st["summ"], st["nsum"], Hq=w.Hq,
                                  enable_gqa=True)

    straight = []
    st = fresh_state()
    run(st, 0, 256, straight)
    torch.cuda.synchronize()
    ref_state = {n: t.cpu() for n, t in st.items()}
    ref_out = torch.stack(straight).cpu()
    del st, straight

    resumed = []
    st = fresh_state()
    run(st, 0, 128, resumed)
    torch.cuda.synchronize()
    saved = {n: t.cpu().clone() for n, t in st.items()}     # to the host
    first = [o.cpu() for o in resumed]
    del st, resumed
    torch.cuda.empty_cache()
    st = {n: t.cuda() for n, t in saved.items()}             # restored
    second = []
    run(st, 128, 256, second)
    torch.cuda.synchronize()
    got = torch.stack(first + [o.cpu() for o in second])
    assert torch.equal(got, ref_out)
    for n in ref_state:
        assert torch.equal(st[n].cpu(), ref_state[n]), n
    assert st["nsum"].cpu().tolist() == [(w.T + 256) // 64] * B
    # and the resumed steps equal the oracle's decode at two of them
    o_summ = O.chunk_summaries(x["k_cache"], x["head_cls"], 1.0 / np.sqrt(D))
    for s in (128, 255):
        L = w.T + 1 + s
        ref = O.decode_step(x["q_steps"][s], x["k_cache"], x["v_cache"], np.full(B, L), o_summ)
        compare_out(got[s].float().numpy(), ref["out"], "bf16", what=f"resumed step {s}")


def test_append_length_beyond_capacity(dash):
    """An append with a length beyond the cache capacity summarises only the chunks inside
    the cache and leaves the summarised-chunk count at most the capacity's chunk count."""
    w = Workload(name="app_cap", kind="prefill", B=2, Hq=8, Hkv=2, T=640, D=128,
                 dtype="bf16", seed=556, needle_amp=1.0)
    x = synth.prefill_inputs(w)
    k, hc = to_dev(x["k"], "bf16"), to_dev(x["head_cls"], "bf16")
    summ = torch.zeros((2, 2, 10, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(2, dtype=torch.int32, device="cuda")
    lens = torch.tensor([640 + 500, 300], dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens, summ, nsum, Hq=8, enable_gqa=True)
    torch.cuda.synchronize()
    assert nsum.cpu().tolist() == [10, 4]
    ref = O.chunk_summaries(x["k"], x["head_cls"], 1.0 / np.sqrt(128))
    got = summ.cpu().numpy()
    np.testing.assert_allclose(got[0], ref[0], atol=2e-5, rtol=1e-5)
    np.testing.assert_allclose(got[1, :, :4], ref[1, :, :4], atol=2e-5, rtol=1e-5)
    assert not got[1, :, 4:].any()
