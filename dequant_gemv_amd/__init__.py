"""Fused dequantise + GEMV (batch 1) for AMD Instinct MI355X (gfx950).

``y = x . dequant(W)^T`` for one activation row over three block formats
(Q4_K, NVFP4 W4A16, TQ1_0).  The compute runs in hand-written HIP kernels in
``libqgemv.so`` behind a C ABI (``include/qgemv.h``); ``dequant_gemv_amd.qgemv``
is the thin Python binding over it.  Nothing is imported eagerly so that the
input generators in ``dequant_gemv_amd.synth`` load without a GPU.
"""

__all__ = ["qgemv", "synth"]
