"""MI355X-native HSTU jagged pointwise attention (libhstu).

The compute path is the HIP library ``libhstu.so`` behind the C ABI declared in
``include/hstu.h``. ``hstu_jagged_pointwise_amd.ops`` is the thin ctypes binding
to it; import it explicitly. It raises if the library has not been built.
``hstu_jagged_pointwise_amd.synth`` holds the seeded input generators and
needs no GPU.
"""
__version__ = "0.1.0"
