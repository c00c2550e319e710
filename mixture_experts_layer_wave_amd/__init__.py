"""Sparse Mixture-of-Experts layer forward for AMD Instinct MI355X (gfx950).

The compute lives in ``libmoe_mi355x.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/moe.h``).  This package holds the thin ctypes
binding (:mod:`.binding`), the build step (:mod:`.build`) and the seeded
synthetic input generators (:mod:`.workloads`).  The binding is imported
lazily so that the generators can be used on machines without the library;
calling any entry point without the built library raises.
"""

_BINDING_NAMES = (
    "moe_abi_version",
    "moe_status_string",
    "moe_workspace_bytes",
    "moe_router_topk",
    "moe_dispatch",
    "moe_grouped_ffn",
    "moe_expert_up",
    "moe_expert_down",
    "moe_combine",
    "moe_forward",
    "MoeError",
    "Shape",
    "ExpertWeights",
    "lib",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
