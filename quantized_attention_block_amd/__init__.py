"""MI355X (gfx950) quantized attention: SageAttention2-style INT8/MXFP4 QK,
FP8 PV and an FP8 paged-KV decode, behind the C ABI of include/sage.h.

The Python API (sage.py) only marshals arguments to libsage.so; build it with
`python -m quantized_attention_block_amd.build`.
"""
from . import sage  # noqa: F401
from .sage import (QK_INT8, QK_MXFP4, Hadamard, SageError, sage_attention,  # noqa: F401
                   sage_attn_fwd, sage_debug_qk_tile, sage_decode_num_splits, sage_paged_decode,
                   sage_quantize_qk, sage_quantize_v)
