"""MI355X (gfx950) split-K decode attention: a C-ABI HIP library plus a thin binding.

The library (libdecode_attention.so, built from csrc/ by build.py) exports the
entry points declared in include/decode_attention.h; ``binding`` wraps them with
the same names for PyTorch tensors.  Import ``decode_attention_07_amd.binding``
to use it; importing this package loads nothing.
"""
