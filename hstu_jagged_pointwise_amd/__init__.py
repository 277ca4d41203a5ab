"""MI355X-native HSTU jagged pointwise attention (libhstu).

The compute path is the HIP library ``libhstu.so`` behind the C ABI declared in
``include/hstu.h``. ``hstu_jagged_pointwise_amd.ops`` is a thin ctypes binding to
it. ``hstu_jagged_pointwise_amd.synth`` holds the seeded input generators. The
binding is imported lazily, so the generators work on a machine without the
library.
"""
__version__ = "0.1.0"


def __getattr__(name):
    if name == "ops":
        from . import ops
        return ops
    raise AttributeError(name)
