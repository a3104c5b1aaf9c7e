"""MI355X-native hierarchical sparse attention (Light Forcing) for chunk-wise
autoregressive video diffusion.

The compute lives in a HIP library (``liblf.so``, C ABI declared in
``include/lf.h``); ``block_sparse_attention_lf_amd.lf`` is the thin ctypes
binding over it. Importing this package does not load the library.
"""
