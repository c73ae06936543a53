"""qblk: block-quantized GEMV/GEMM for MI355X (gfx950).

The C-ABI library is loaded on first use of a binding function
(``block_quantized_qblk_amd.qblk``); importing the package itself loads
nothing, so ``block_quantized_qblk_amd.synth`` can be used on its own.
"""

__all__ = ["qblk", "synth"]
