"""Batch-invariant transformer forward kernels for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libbi.so`` (hand-written HIP kernels);
``invariant_bi_rmsnorm_amd.ops`` is its thin ctypes binding.  Importing this
package does not load the library; ``ops`` does, and fails loudly when the
library is missing.
"""
__all__ = ["ops", "inputs"]
