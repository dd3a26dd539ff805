"""MI355X-native staged decode attention for beam-search generative recommendation.

The compute path is the C-ABI library ``libxattn.so`` (hand-written HIP
kernels for gfx950, declared in ``include/xattn.h``); this package is its
thin Python binding.  The binding loads the library on first use and raises
if it is missing: there is no fallback implementation.
"""
from . import workloads  # noqa: F401  (seeded inputs; no attention arithmetic)

_BINDING = ("decode", "decode_noalloc", "decode_with_ancestors", "decode_per_beam", "decode_debug",
            "resolve_ancestors", "workspace_size", "plan", "make_shape", "Shape",
            "beam_topk", "reorder_unshared", "trie_build", "ValidPaths", "library_path",
            "XattnError", "PreparedDecode", "load")
__all__ = list(_BINDING[:-1]) + ["workloads"]


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
