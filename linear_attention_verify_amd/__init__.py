"""MI355X-native GatedDeltaNet speculative verify/commit.

The compute lives in a HIP library (``libgdn_spec.so``, built from ``csrc/``
for gfx950) behind the C ABI declared in ``include/gdn_spec.h``; ``binding``
marshals torch tensors onto it. ``workloads`` draws seeded synthetic inputs.
The binding is imported lazily so that drawing inputs never loads the GPU library.
"""

__all__ = ["binding", "workloads", "build"]


def __getattr__(name):
    if name in ("binding", "build"):
        import importlib
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
