"""MI355X (gfx950) implementation of the Recurrent Looped Transformer's
batched recurrent decoder state transition.

The compute path is ``librlt.so`` (hand-written HIP kernels behind the C ABI
in ``include/rlt.h``); ``_abi`` mirrors that ABI with ctypes and ``runtime``
manages device buffers with PyTorch. Build with
``python -m stateful_sequence_model_amd.build``; calls raise if the library
is missing.
"""
from . import _abi  # noqa: F401
from .runtime import Decoder, DecoderState, MemoryWeights, ModelConfig, current_stream, to_device  # noqa: F401

__all__ = ["Decoder", "DecoderState", "MemoryWeights", "ModelConfig", "current_stream", "to_device"]
