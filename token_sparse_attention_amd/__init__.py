"""MI355X-native MC-Sparse token-sparse attention.

The compute path is the C-ABI library ``libmcs.so`` (hand-written HIP kernels
for gfx950, declared in include/mcs.h).  ``binding`` marshals torch tensors to
it; nothing in this package computes attention on the CPU.
"""
__version__ = "0.1.0"
