"""MI355X (gfx950) DF-SSM scaffold projection: 1-bit sign-packed weights x per-token
int8 activations, int32 accumulation, fused int8 rank-16 LoRA epilogue.

The compute lives in the HIP library ``libdfssm.so`` (C ABI in ``include/dfssm.h``);
``bit_scaffold_int8_amd.dfssm`` is its thin ctypes binding.  Import that module to
use the library; it raises ImportError when the library has not been built.
"""
__all__ = ["dfssm"]
