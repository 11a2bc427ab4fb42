"""USP (Ulysses + zigzag Ring-Attention) forward hot path for AMD MI355X.

The compute lives in ``libusp.so`` (hand-written HIP kernels for gfx950,
C ABI in ``include/usp.h``); ``binding`` marshals torch tensors into it and
``inputs`` draws the seeded synthetic workloads.  The binding is loaded on
first use, so ``inputs`` can be imported on machines without the library.
"""
_BINDING_NAMES = {"usp_zigzag_extract", "usp_ulysses_a2a_layout", "usp_ring_attn_step_fwd",
                  "usp_lse_merge", "usp_attn_fwd", "attn_desc", "UspError", "UspAttnDesc", "lib"}


_API_NAMES = {"zigzag_extract", "attn", "rank_to_grid"}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    if name in _API_NAMES:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
