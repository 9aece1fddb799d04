"""DashAttention forward pass for MI355X (gfx950): C-ABI HIP library + thin binding.

    from long_context_sparse_stage0_amd import dash
    out = dash.prefill(q, k, v, head_cls, alpha=1.5, enable_gqa=True)

The binding module is imported lazily so that the input generator and the workload
definitions stay importable on machines without the built library.
"""
__all__ = ["dash", "synth", "workloads"]
