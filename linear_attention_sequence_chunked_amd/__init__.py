"""MI355X (gfx950) Kimi Delta Attention: chunked prefill and decode step.

The compute runs in libkda.so (hand-written HIP kernels behind the C ABI of
include/kda.h); this package only marshals torch tensors and the current stream.
"""
from ._lib import KdaError, LIB_PATH, load as load_library  # noqa: F401
from .ops import (checkpoint_slot, chunk_prefill, chunk_prefill_segmented,  # noqa: F401
                  decode_step, prefill_backward, spec_commit, spec_verify)

__all__ = ["chunk_prefill", "chunk_prefill_segmented", "checkpoint_slot", "prefill_backward", "decode_step", "spec_verify", "spec_commit",
           "KdaError", "load_library", "LIB_PATH"]
