"""MI355X-native decode-phase paged attention.

The compute path is the HIP library ``libdecode_attn.so`` (kernels for gfx950
behind a C ABI declared in ``include/decode_attn.h``); ``binding`` marshals
torch tensors into that ABI. ``workload`` draws seeded synthetic inputs.

The binding is imported lazily so that the workload generator can be used on
a machine where the library has not been built.
"""

__all__ = ["decode_attn", "decode_attn_ex", "decode_attn_append", "decode_attn_prefill", "plan",
           "binding", "workload"]


def __getattr__(name):
    if name in ("decode_attn", "decode_attn_ex", "decode_attn_append", "decode_attn_prefill", "plan"):
        from . import binding
        return getattr(binding, name)
    if name in ("binding", "workload"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
