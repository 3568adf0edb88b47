"""MI355X-native fused equivariant message-passing convolution (gfx950 HIP).

The compute path lives in the C-ABI library ``libe3hip.so`` (kernels under
``csrc/``); ``api`` is its thin Python binding and ``synth`` the seeded input
generator.  Importing the package loads nothing: the library is opened on the
first call into ``api``.
"""
__all__ = ["api", "synth"]
