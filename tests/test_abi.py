"""The C-ABI library loads, exports every entry point its header declares, and rejects bad
arguments on the host (CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dash.h")

dash = pytest.importorskip("long_context_sparse_stage0_amd.dash")


def _lib():
    if not os.path.exists(dash.LIB_PATH):
        pytest.skip("libdash.so not built (run __graft_entry__.build())")
    return dash.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(dash.EXPORTS)


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    assert lib.dash_abi_version() == 105


FAKE = ctypes.c_void_p(1 << 20)        # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)


def _params(**kw):
    base = dict(B=1, Hq=4, Hkv=2, T=256, D=128, chunk_size=64, alpha=1.5, gamma=1.0,
                sm_scale=0.0, enable_gqa=1, dtype=0, estimate_diagonal=0, sigma=1.0, topk=0)
    base.update(kw)
    return dash.DashParams(**base)


def _ws(p):
    n = ctypes.c_size_t(0)
    rc = _lib().dash_prefill_workspace_size(ctypes.byref(p), ctypes.byref(n))
    return rc, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), -2),                    # Hq % Hkv != 0
    (dict(Hq=4, Hkv=2, enable_gqa=0), -2),      # GQA shape without the flag
    (dict(Hq=12, Hkv=4), -4),                   # 3 heads per KV head: not built
    (dict(Hq=64, Hkv=2), -4),                   # 32 heads per KV head: not built
    (dict(D=96), -4),
    (dict(chunk_size=128), -4),
    (dict(alpha=1.0), -1),
    (dict(alpha=0.5), -1),
    (dict(alpha=float("nan")), -1),
    (dict(alpha=float("inf")), -1),
    (dict(gamma=0.0), -1),
    (dict(sm_scale=float("inf")), -1),
    (dict(T=0), -1),
    (dict(T=-5), -1),
    (dict(B=0), -1),
    (dict(dtype=7), -3),
    (dict(sigma=-0.5), -1),
    (dict(sigma=float("nan")), -1),
    (dict(sigma=float("inf")), -1),
    (dict(topk=-1), -1),
    (dict(T=64 * 2049 + 1), -4),
])
def test_param_validation(kw, code):
    lib = _lib()
    p = _params(**kw)
    rc, _ = _ws(p)
    assert rc == code, lib.dash_last_error()
    assert lib.dash_last_error().decode()
    rc = lib.dash_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None,
                          FAKE, 1 << 40, None)
    assert rc == code


def test_valid_params_and_workspace_sizes():
    lib = _lib()
    rc, n = _ws(_params())
    assert rc == 0 and n > 0 and lib.dash_last_error() == b""
    # 128K tokens, 32 query / 2 KV heads, bf16: summaries, V^T, mask and weights fit easily
    rc, n = _ws(_params(B=1, Hq=32, Hkv=2, T=131072, D=128))
    assert rc == 0
    assert 2 * 2 ** 30 < n < 3 * 2 ** 30
    rc, n = _ws(_params(T=64 * 2049))           # the longest supported sequence
    assert rc == 0


def test_pointer_and_workspace_validation():
    lib = _lib()
    p = _params()
    rc, need = _ws(p)
    assert rc == 0
    args = [FAKE] * 5
    for i in range(5):
        bad = list(args)
        bad[i] = None
        assert lib.dash_prefill(ctypes.byref(p), *bad, None, None, None, FAKE, need, None) == -1
        bad[i] = MISALIGNED
        assert lib.dash_prefill(ctypes.byref(p), *bad, None, None, None, FAKE, need, None) == -1
    assert lib.dash_prefill(ctypes.byref(p), *args, MISALIGNED, None, None, FAKE, need, None) == -1
    assert lib.dash_prefill(ctypes.byref(p), *args, None, None, None, None, need, None) == -5
    assert lib.dash_prefill(ctypes.byref(p), *args, None, None, None, FAKE, need - 1, None) == -5
    assert lib.dash_prefill(ctypes.byref(p), *args, None, None, None,
                            ctypes.c_void_p((1 << 20) + 16), need, None) == -1
    assert b"workspace" in lib.dash_last_error() or b"aligned" in lib.dash_last_error()
    assert lib.dash_prefill(None, *args, None, None, None, FAKE, need, None) == -1


def test_decode_append_dense_validation():
    lib = _lib()
    p = _params(T=65792, Hq=32, Hkv=2)
    n = ctypes.c_size_t(0)
    assert lib.dash_decode_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert n.value > 0
    # NULL seq_lens
    assert lib.dash_decode(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                           n.value, None) == -1
    assert lib.dash_decode(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           0, None) == -5
    assert lib.dash_append_chunk(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.dash_append_chunk(ctypes.byref(_params(alpha=1.0)), FAKE, FAKE, FAKE, FAKE,
                                 FAKE, None) == -1
    # paged caches: a block table is required, the pool must be non-empty, bf16 only
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 4, None, FAKE, FAKE, FAKE,
                                 None, FAKE, n.value, None) == -1
    assert lib.dash_decode_paged(ctypes.byref(p), FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, n.value, None) == -1
    assert lib.dash_decode_paged(ctypes.byref(_params(dtype=1)), FAKE, FAKE, FAKE, 4, FAKE,
                                 FAKE, FAKE, FAKE, None, FAKE, n.value, None) == -4
    assert lib.dash_append_chunk_paged(ctypes.byref(p), FAKE, 4, None, FAKE, FAKE, FAKE, FAKE,
                                       None) == -1
    assert lib.dash_append_chunk_paged(ctypes.byref(p), FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       None) == -1
    # the top-k comparison router: bf16 only
    pt = _params(T=65792, Hq=32, Hkv=2, topk=8, dtype=1)
    assert lib.dash_decode(ctypes.byref(pt), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           1 << 30, None) == -4
    assert lib.dash_prefill(ctypes.byref(_params(dtype=1, topk=8)), FAKE, FAKE, FAKE, FAKE,
                            FAKE, None, None, None, FAKE, 1 << 30, None) == -4
    # estimate_diagonal: entmax prefill only, at most 2048 chunks per sequence
    for kw in (dict(dtype=0, topk=4), dict(dtype=1, T=64 * 2048 + 1), dict(dtype=0, T=64 * 2049)):
        pe = _params(estimate_diagonal=1, **kw)
        assert lib.dash_prefill(ctypes.byref(pe), FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                None, FAKE, 1 << 40, None) == -4, kw
    # decode: the flag needs head_cls (dash_decode_diag); not with paged caches or top-k
    pe = _params(estimate_diagonal=1, dtype=1)
    assert lib.dash_decode(ctypes.byref(pe), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                           1 << 30, None) == -1
    assert lib.dash_decode_diag(ctypes.byref(pe), FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                None, FAKE, 1 << 30, None) == -1
    assert lib.dash_decode_diag(ctypes.byref(pe), FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE,
                                FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.dash_decode_diag(ctypes.byref(_params(estimate_diagonal=1, topk=3)), FAKE, FAKE,
                                FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == -4
    assert lib.dash_decode_paged(ctypes.byref(_params(estimate_diagonal=1)), FAKE, FAKE, FAKE,
                                 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == -1
    assert lib.dash_decode_paged_diag(ctypes.byref(_params(estimate_diagonal=1)), FAKE, FAKE,
                                      FAKE, 4, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                                      None) == -1
    assert lib.dash_decode_paged_diag(ctypes.byref(_params(estimate_diagonal=1, dtype=1)), FAKE,
                                      FAKE, FAKE, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                      1 << 30, None) == -4
    # the dense comparator is bf16 only
    pf = _params(dtype=1)
    assert lib.dash_dense_causal_workspace_size(ctypes.byref(pf), ctypes.byref(n)) == -3
    assert lib.dash_dense_causal(ctypes.byref(_params()), FAKE, None, FAKE, FAKE, FAKE,
                                 1 << 30, None) == -1


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    saved = dash._lib
    try:
        dash._lib = None
        with pytest.raises(RuntimeError, match="libdash.so not found"):
            dash.load(str(tmp_path / "missing.so"))
    finally:
        dash._lib = saved


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it exits with a message before touching
    torch or a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_prefill_stage_index_validation():
    """dash_prefill_stage takes stage 0 (summaries), 1 (routing), 2 (attention) or 3 (the
    chunk-transposed V copy); anything else is rejected before any launch."""
    lib = _lib()
    p = _params()
    rc, need = _ws(p)
    for stage in (-1, 4, 7):
        assert lib.dash_prefill_stage(ctypes.byref(p), stage, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      None, None, None, FAKE, need, None) == -1
        assert b"stage" in lib.dash_last_error()


def test_decode_noalloc_rejects_oversize_on_host():
    """dash_decode_noalloc checks the shape's scratch need against its fixed array before any
    HIP call: an oversize shape is DASH_ERR_WORKSPACE even without a GPU."""
    lib = _lib()
    p = _params(B=64, Hq=32, Hkv=2, T=64 * 2049)
    rc = lib.dash_decode_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert rc == -5
    assert b"scratch" in lib.dash_last_error()
    assert lib.dash_decode_noalloc(ctypes.byref(_params(alpha=1.0)), FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, None, None) == -1
