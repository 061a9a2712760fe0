"""Ragged pack -> attend -> unpack for token-pruned ViTs on AMD MI355X (gfx950).

The compute path is librag.so (hand-written HIP kernels behind a C ABI, see
include/rag.h); ``binding`` marshals torch GPU tensors into it.  ``workloads``
draws seeded synthetic DeiT-shaped inputs.  The binding is imported lazily so
that the workload generator can be used without the GPU library.
"""
__all__ = ["binding", "workloads", "build"]


def __getattr__(name):
    if name in ("rag_pack", "rag_repack", "rag_attn", "rag_attn_tiled", "rag_unpack", "rag_attn_padded", "rag_attn_gathered",
                "Pipeline", "Block", "RagError", "last_error"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
