"""One layer of Qwen Sparse Attention (QSA) on MI355X (gfx950).

The compute lives in the HIP library ``libqsa.so`` built from ``csrc/``; the
Python module ``qsa`` only marshals tensors and streams into its C ABI.
Importing this package loads nothing; ``qsa.lib()`` loads the library and
raises if it has not been built.
"""

__all__ = ["inputs", "qsa"]
