"""Named synthetic workloads (shapes, dtypes and generator settings only).

The pages measure prefill at 16K/75% and 96K/93.7% sparsity and decoding at 96K with
batch 24 (liuzhao09 reading note, section 3, Table 5; aixai.ru blog, section
"Эксперименты: точность и скорость").  Their accuracy suites are not available, so the
workloads below are seeded synthetic stand-ins of comparable length, with planted
"needle" chunks (reading note, section 6: validate needle recovery on synthetic
retrieval data first).

Nothing here computes any part of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

CHUNK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    T: int                    # prefill: sequence length; decode: tokens already in the cache
    D: int
    dtype: str                # "bf16" or "fp32"
    alpha: float = 1.5
    gamma: float = 1.0
    seed: int = 0
    q_mode: str = "coherent"  # "iid" or "coherent" (block-coherent queries)
    coherence_j: float = 0.25
    needle_count: str = "uniform32"   # "none", "uniform32", "poisson"
    needle_lambda: float = 0.0
    needle_amp: float = 3.0
    head_cls_std: float = 1.0 / 8.0
    steps: int = 0            # decode only: new tokens per sequence

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def enable_gqa(self) -> bool:
        return self.Hq != self.Hkv

    @property
    def T_total(self) -> int:
        """Capacity needed: prefill T, decode cache T + steps."""
        return self.T + self.steps

    def scaled(self, T: int, **kw) -> "Workload":
        """Same heads, head_dim and generator, shorter sequence (parity-size copy)."""
        return replace(self, T=T, name=f"{self.name}@T{T}", **kw)


# Amplitude of the needle shift for the 128K workload, chosen by
# oracle/calibrate_needles.py so that about 75% of causal (row, kv-head, chunk) pairs
# receive zero routing weight.  The 64K decode and sweep workloads reuse it.
CALIBRATED_AMP = 0.328125

PREFILL_1K_FP32 = Workload(
    name="prefill_1k_fp32", kind="prefill", B=1, Hq=2, Hkv=2, T=1024, D=64,
    dtype="fp32", seed=20260001, q_mode="iid", needle_count="none")

PREFILL_16K_GQA = Workload(
    name="prefill_16k_gqa32x8", kind="prefill", B=1, Hq=32, Hkv=8, T=16384, D=128,
    dtype="bf16", seed=20260002, needle_count="uniform32", needle_amp=3.0)

PREFILL_128K_GQA = Workload(
    name="prefill_128k_gqa32x2", kind="prefill", B=1, Hq=32, Hkv=2, T=131072, D=128,
    dtype="bf16", seed=20260003, needle_count="uniform32", needle_amp=CALIBRATED_AMP)

DECODE_64K_B16 = Workload(
    name="decode_64k_b16", kind="decode", B=16, Hq=32, Hkv=2, T=65536, D=128,
    dtype="bf16", seed=20260004, needle_count="uniform32", needle_amp=CALIBRATED_AMP,
    steps=256)


def sweep_cell(alpha: float, lam: float) -> Workload:
    ia = {1.25: 0, 1.5: 1, 2.0: 2}[alpha]
    il = {2.0: 0, 8.0: 1, 32.0: 2}[lam]
    return Workload(
        name=f"sweep_64k_gqa32x8_a{alpha}_l{int(lam)}", kind="prefill", B=1, Hq=32, Hkv=8,
        T=65536, D=128, dtype="bf16", alpha=alpha, seed=20265000 + 10 * ia + il,
        needle_count="poisson", needle_lambda=lam, needle_amp=CALIBRATED_AMP)


SWEEP = [sweep_cell(a, l) for a in (1.25, 1.5, 2.0) for l in (2.0, 8.0, 32.0)]

ALL = {w.name: w for w in [PREFILL_1K_FP32, PREFILL_16K_GQA, PREFILL_128K_GQA, DECODE_64K_B16] + SWEEP}
