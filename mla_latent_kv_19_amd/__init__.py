"""MI355X-native multi-head latent attention (MLA) over the latent KV cache.

The compute lives in ``libmla.so`` (hand-written HIP for gfx950) behind a
C ABI; ``mla_latent_kv_19_amd.api`` is the thin torch binding over it and
``mla_latent_kv_19_amd.synth`` draws seeded synthetic inputs.  Importing this
package loads nothing; the library is loaded on first use of ``api``.
"""

__all__ = ["api", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
