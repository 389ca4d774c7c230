"""MI355X-native equivariant edge convolution.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
of ``include/eec.h`` (library ``libeec.so``, built in-tree by
``equivariant_edge_convolution_amd.build``).  ``binding`` is a thin ctypes
layer over it that takes PyTorch device tensors; the library is loaded on first
use and its absence is an error.
"""
