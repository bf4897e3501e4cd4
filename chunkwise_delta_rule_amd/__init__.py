"""libmdn: Momentum DeltaNet chunkwise forward and decode step on MI355X.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
in ``include/libmdn.h``; ``mdn`` is its thin Python binding.
"""
from .mdn import (CHUNK, ChunkPlan, GateParams, HEAD_DIMS, MDN_BF16, MDN_F32, MdnError, chunk_bwd,
                  chunk_fwd, decode_step, gates_from_logits, load_library, output_epilogue, qk_prologue,
                  workspace_bytes)

__all__ = ["CHUNK", "ChunkPlan", "GateParams", "HEAD_DIMS", "MDN_BF16", "MDN_F32", "MdnError",
           "chunk_bwd", "chunk_fwd", "decode_step", "gates_from_logits", "load_library", "output_epilogue", "qk_prologue",
           "workspace_bytes"]
