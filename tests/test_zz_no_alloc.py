"""dash_decode_noalloc (the decode step on the library's fixed device scratch, for callers
that cannot allocate) against dash_decode with a caller workspace: two calls in a row, the
second with a smaller input, each bit-identical to the workspace path; and a shape whose
scratch would exceed the fixed size is rejected before any launch."""
import numpy as np
import pytest

from long_context_sparse_stage0_amd import synth
from long_context_sparse_stage0_amd.workloads import Workload
from tests.parity_util import say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dash():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_stage0_amd import dash as d
    d.load()
    return d


def _case(dash, B, lens, Hq, T, seed):
    w = Workload(name="noalloc", kind="prefill", B=B, Hq=Hq, Hkv=2, T=T, D=128,
                 dtype="bf16", seed=seed, needle_amp=0.5)
    x = synth.prefill_inputs(w)
    k, v, hc = (to_dev(x[n], "bf16") for n in ("k", "v", "head_cls"))
    nc = -(-T // 64)
    summ = torch.zeros((B, 2, nc, 128), dtype=torch.float32, device="cuda")
    nsum = torch.zeros(B, dtype=torch.int32, device="cuda")
    lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
    dash.append_chunk(k, hc, lens_t, summ, nsum, Hq=Hq, enable_gqa=True)
    q = torch.stack([to_dev(x["q"][b, :, lens[b] - 1], "bf16") for b in range(B)]).contiguous()
    return q, k, v, lens_t, summ, nc


def test_decode_noalloc_matches_workspace_path(dash):
    cases = [dict(B=4, lens=[6000, 4097, 700, 6000], Hq=32, T=6000, seed=71),
             dict(B=2, lens=[1500, 65], Hq=8, T=1500, seed=72)]        # second call: smaller
    for i, c in enumerate(cases):
        say(f"[no-alloc] call {i}: B={c['B']} Hq={c['Hq']} T={c['T']}")
        q, k, v, lens_t, summ, nc = _case(dash, **c)
        W = -(-nc // 64)
        ref, ab_ref = dash.decode(q, k, v, lens_t, summ, enable_gqa=True,
                                  return_active_blocks=True)
        out = torch.empty_like(q)
        ab = torch.empty((c["B"], 2, W), dtype=torch.int64, device="cuda")
        got = dash.decode_noalloc(q, k, v, lens_t, summ, enable_gqa=True, out=out,
                                  active_blocks=ab)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {i}: outputs differ"
        assert torch.equal(ab, ab_ref), f"call {i}: masks differ"
        assert np.isfinite(got.float().cpu().numpy()).all()


def test_decode_noalloc_rejects_oversize(dash):
    """A shape needing more scratch than the fixed array is refused with
    DASH_ERR_WORKSPACE and a message, and nothing is launched."""
    B, Hq, T = 64, 32, 64 * 2049
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dash.DashError, match="scratch"):
        p = dash.make_params(B, Hq, 2, T, 128, enable_gqa=True, dtype=torch.bfloat16)
        import ctypes
        lib = dash.load()
        lens = torch.ones(B, dtype=torch.int32, device="cuda")
        summ = torch.zeros((1, 128), dtype=torch.float32, device="cuda")
        dash._check(lib.dash_decode_noalloc(ctypes.byref(p), dash._ptr(q), dash._ptr(kv),
                                            dash._ptr(kv), dash._ptr(lens), dash._ptr(summ),
                                            dash._ptr(q), None, dash._stream(None)))
