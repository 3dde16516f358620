"""MI355X-native DSA (DeepSeek Sparse Attention) decode path for GLM-5.3-Flash.

The compute lives in ``libdsa.so`` (hand-written gfx950 HIP kernels behind a
C ABI declared in ``include/dsa.h``); ``sparse_attention_fp32_amd.dsa`` is a
thin ctypes binding over it that marshals torch device tensors and streams.
"""
