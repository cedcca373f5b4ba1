"""Attention over a paged KV cache for AMD MI355X (gfx950).

The compute lives in libpagedkv.so (hand-written HIP kernels behind the C ABI
in include/pagedkv.h); ``binding`` marshals torch tensors onto it and
``workloads`` generates seeded synthetic inputs. Importing the package loads
nothing; the library is loaded on the first call.
"""

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in ("paged_kv_write", "paged_attention_decode", "paged_attention_varlen",
                "paged_attention_decode_workspace_size"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
