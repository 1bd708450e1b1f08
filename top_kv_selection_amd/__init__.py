"""CSA2 sparse attention for MI355X: hierarchical block pass, exact token
Top-K and sparse + sliding-window attention in hand-written HIP for gfx950.

``binding`` wraps the C ABI of ``libcsa2.so`` (declared in include/csa2.h);
``pipeline`` runs a workload's layer groups; ``workloads`` draws seeded
synthetic inputs.  Importing ``binding`` (or anything that uses it) fails
loudly if the library has not been built.
"""
__all__ = ["binding", "pipeline", "workloads", "build"]
