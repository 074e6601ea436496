"""Jagged flash attention for MI355X (gfx950): forward and backward on values+offsets tensors.

The compute path is ``libjfa.so`` (hand-written HIP kernels behind the C ABI in include/jfa.h);
this package only marshals arguments to it. Importing ``jagged_sequence_amd.binding`` loads the
library and fails loudly when it is not built.
"""
__all__ = ["binding", "flops"]
